// ring_step.hip -- one decode step of SnapKV's ring-buffer adaptation for
// every KV head (gfx950).
//
// [SNAP] "How it works" and "On the adaptation": each cached token keeps a
// ring of its last obsWindow observed attention weights; an observed step
// writes every cached token's weight at the ring index and advances it (a
// null step writes nothing and does not advance); the new token enters with
// a zero ring; over the budget, the ring sums (index 0 upward) are max-pooled
// over the poolKernel tokens centred on each in position order (clamped) and
// the smallest (pooled, position) outside the recent window is dropped, equal
// scores dropping the lower position.
//
// One 1024-thread workgroup per head:
//   1. block ids to LDS; the append's block (popped from the free list when
//      its logical block has none);
//   2. logits of the G query rows against every cached key and the new key
//      (a 16-byte piece of the key row per lane, lanes of a token reduced by
//      shuffles), in log2 units, in LDS;
//   3. each row's log-sum-exp2;
//   4. per cached slot: the weight (group sum of the probabilities), written
//      at the ring index; at the budget the ring sum; the count of cached
//      positions below the new token's (its rank);
//   5. at the budget: the sums laid out in position order through the
//      persistent per-slot ranks, the pooled maximum, and the packed
//      (score key, position) minimum over the candidates;
//   6. the writes: the new token's K/V row, position and zero ring into the
//      append slot or the victim's slot, and every slot's rank.
// Ranks make position order available without a sort: they are kept as each
// slot's index in position order and updated in one parallel pass.
#include <hip/hip_runtime.h>

#include "kvev_device.h"
#include "kvev_kernels.h"

namespace kvev {

namespace {
constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / kWave;

template <bool BF16>
__device__ __forceinline__ float dot_piece(uint4 a, uint4 b) {
  if constexpr (BF16) {
    const uint32_t x[4] = {a.x, a.y, a.z, a.w}, y[4] = {b.x, b.y, b.z, b.w};
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      s = fmaf(__uint_as_float(x[i] << 16), __uint_as_float(y[i] << 16), s);
      s = fmaf(__uint_as_float(x[i] & 0xffff0000u), __uint_as_float(y[i] & 0xffff0000u), s);
    }
    return s;
  } else {
    float s = __uint_as_float(a.x) * __uint_as_float(b.x);
    s = fmaf(__uint_as_float(a.y), __uint_as_float(b.y), s);
    s = fmaf(__uint_as_float(a.z), __uint_as_float(b.z), s);
    s = fmaf(__uint_as_float(a.w), __uint_as_float(b.w), s);
    return s;
  }
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = kWave / 2; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = kWave / 2; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ int wave_sum_i(int v) {
#pragma unroll
  for (int o = kWave / 2; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ uint64_t wave_min_u64(uint64_t v) {
#pragma unroll
  for (int o = kWave / 2; o >= 1; o >>= 1) {
    const uint64_t w = (uint64_t)__shfl_xor((unsigned long long)v, o);
    v = w < v ? w : v;
  }
  return v;
}
}  // namespace

// LPT: lanes per token (row_bytes / 16); G <= kRingMaxGroup.
template <bool BF16, int LPT>
__global__ __launch_bounds__(kThreads) void ring_step_kernel(const RingArgs P) {
  extern __shared__ __align__(16) float lds[];
  __shared__ int s_bt[kRingMaxBlocks];
  __shared__ int s_code, s_blk, s_bad, s_victim;
  __shared__ int s_cnt[kWaves];
  __shared__ float s_red[kWaves][kRingMaxGroup];
  __shared__ float s_lse[kRingMaxGroup];
  __shared__ unsigned long long s_min[kWaves];
  constexpr int TPW = kWave / LPT;  // tokens per wave pass
  const int u = blockIdx.x, b = u / P.Hkv, tid = threadIdx.x, l = lane_id(), wv = tid / kWave;
  const int G = P.G, W = P.W, ms = P.max_slots;
  const int n = P.seq_len[u], t = P.t_pos[b];
  const int ring0 = P.ring[u];
  const bool observe = P.observe[b] != 0;
  int32_t *bt = P.block_table + (size_t)u * P.max_blocks;
  int32_t *ps = P.pos + (size_t)u * ms;
  int32_t *rk = P.rank + (size_t)u * ms;
  float *hs = P.hist + (size_t)u * W * ms;
  if (n < 0 || n > P.budget || ring0 < 0 || ring0 >= W) {
    if (tid == 0) P.evicted[u] = -2;
    return;
  }
  const int nb = (n + kBlock - 1) / kBlock;
  if (tid == 0) s_bad = 0;
  __syncthreads();
  for (int lb = tid; lb < nb; lb += kThreads) {
    const int e = bt[lb];
    s_bt[lb] = e;
    if (e < 0 || e >= P.num_blocks) s_bad = 1;
  }
  // ranks outside [0, n) (not left by the ring step or its init): refused
  for (int j = tid; j < n; j += kThreads)
    if ((unsigned)P.rank[(size_t)u * ms + j] >= (unsigned)n) s_bad = 2;
  __syncthreads();
  if (s_bad == 2) {
    if (tid == 0) P.evicted[u] = -2;
    return;
  }
  const bool append = n < P.budget;
  if (tid == 0) {
    int code = s_bad ? -4 : 0, blk = -1;
    if (!code && append) {
      const int e = bt[n / kBlock];
      if (e >= P.num_blocks || (e < 0 && n % kBlock != 0)) {
        code = -4;
      } else if (e >= 0) {
        blk = e;
      } else {  // the append opens a block: one from the top of the free list
        const int old = atomicSub(P.free_count, 1);
        if (old <= 0) {
          atomicAdd(P.free_count, 1);
          code = -3;
        } else {
          blk = P.free_list[old - 1];
          if (blk < 0 || blk >= P.num_blocks) code = -4;  // a bad entry stays taken
          else bt[n / kBlock] = blk;
        }
      }
    }
    s_code = code;
    s_blk = blk;
  }
  __syncthreads();
  if (s_code) {
    if (tid == 0) P.evicted[u] = s_code;
    return;
  }
  const int row_bytes = LPT * 16;
  const int np = P.budget + 1;  // logits row stride
  float *lg = lds;              // [G][np] logits (log2 units), then the position-ordered sums
  float *ord = lds + (size_t)G * np;
  // 2. logits: a wave takes TPW tokens a pass, LPT lanes each
  {
    const int piece = l % LPT, tw = l / LPT;
    uint4 qv[kRingMaxGroup];
#pragma unroll
    for (int g = 0; g < kRingMaxGroup; ++g)
      if (g < G)
        qv[g] = ld16(P.q + ((size_t)u * G + g) * row_bytes + piece * 16);
    for (int j0 = wv * TPW; j0 <= n; j0 += kWaves * TPW) {
      const int j = j0 + tw;
      const bool valid = j <= n;
      uint4 kv = make_uint4(0, 0, 0, 0);
      bool masked = !valid;
      if (valid) {
        if (j < n) {
          masked = ps[j] > t;
          const size_t row = (size_t)s_bt[j / kBlock] * kBlock + j % kBlock;
          kv = ld16(P.k_pool + row * row_bytes + piece * 16);
        } else {
          kv = ld16(P.k_new + (size_t)u * row_bytes + piece * 16);
        }
      }
#pragma unroll
      for (int g = 0; g < kRingMaxGroup; ++g) {
        if (g >= G) break;
        float d = dot_piece<BF16>(qv[g], kv);
#pragma unroll
        for (int o = LPT / 2; o >= 1; o >>= 1) d += __shfl_xor(d, o);
        if (valid && piece == 0) lg[g * np + j] = masked ? -__builtin_inff() : d * P.c1;
      }
    }
  }
  __syncthreads();
  // 3. each row's log-sum-exp2 over the n + 1 logits
  for (int g = 0; g < G; ++g) {
    float m = -__builtin_inff();
    for (int j = tid; j <= n; j += kThreads) m = fmaxf(m, lg[g * np + j]);
    m = wave_max(m);
    if (l == 0) s_red[wv][g] = m;
  }
  __syncthreads();
  if (tid < G) {
    float m = -__builtin_inff();
    for (int w = 0; w < kWaves; ++w) m = fmaxf(m, s_red[w][tid]);
    s_lse[tid] = m;
  }
  __syncthreads();
  for (int g = 0; g < G; ++g) {
    const float m = s_lse[g];
    float z = 0.f;
    for (int j = tid; j <= n; j += kThreads) z += __builtin_amdgcn_exp2f(lg[g * np + j] - m);
    z = wave_sum(z);
    if (l == 0) s_red[wv][g] = z;
  }
  __syncthreads();
  if (tid < G) {
    float z = 0.f;
    for (int w = 0; w < kWaves; ++w) z += s_red[w][tid];
    s_lse[tid] = s_lse[tid] + __builtin_amdgcn_logf(z);  // log2
  }
  __syncthreads();
  // 4. weights into the rings; the sums; the new token's rank
  const int r = (P.pool_kernel - 1) / 2;
  int below = 0;
  for (int j = tid; j < n; j += kThreads) {
    float w = 0.f;
    for (int g = 0; g < G; ++g) w += __builtin_amdgcn_exp2f(lg[g * np + j] - s_lse[g]);
    if (observe) hs[(size_t)ring0 * ms + j] = w;
    below += ps[j] < t ? 1 : 0;
    if (!append) {  // the ring sum, index 0 upward; kept in this slot's first logit
      float acc = 0.f;
      for (int q = 0; q < W; ++q) acc += (observe && q == ring0) ? w : hs[(size_t)q * ms + j];
      lg[j] = acc;
    }
  }
  below = wave_sum_i(below);
  if (l == 0) s_cnt[wv] = below;
  __syncthreads();
  int new_rank = 0;
  for (int w = 0; w < kWaves; ++w) new_rank += s_cnt[w];
  if (tid == 0 && observe) P.ring[u] = ring0 + 1 == W ? 0 : ring0 + 1;
  // 5. at the budget: position-ordered sums, pooling, the victim
  int victim = -1;  // slot, n for the new token
  if (!append) {
    for (int j = tid; j < n; j += kThreads) {
      const int rj = rk[j];
      ord[rj + (rj >= new_rank ? 1 : 0)] = lg[j];
    }
    if (tid == 0) ord[new_rank] = 0.f;
    __syncthreads();
    uint64_t best = ~0ull;
    for (int j = tid; j <= n; j += kThreads) {
      const int pj = j < n ? ps[j] : t;
      if (t - pj < P.recent) continue;
      const int cr = j < n ? rk[j] + (rk[j] >= new_rank ? 1 : 0) : new_rank;
      const int lo = max(0, cr - r), hi = min(n, cr + r);
      float m = ord[lo];
      for (int k = lo + 1; k <= hi; ++k) m = fmaxf(m, ord[k]);
      const uint64_t key = ((uint64_t)score_key(m) << 32) | (uint32_t)(pj ^ 0x80000000);
      best = key < best ? key : best;
    }
    best = wave_min_u64(best);
    if (l == 0) s_min[wv] = best;
    if (tid == 0) s_victim = -1;
    __syncthreads();
    uint64_t mn = ~0ull;
    for (int w = 0; w < kWaves; ++w) mn = s_min[w] < mn ? s_min[w] : mn;
    if (mn != ~0ull) {
      const int vpos = (int)((uint32_t)mn ^ 0x80000000u);
      for (int j = tid; j <= n; j += kThreads) {
        const int pj = j < n ? ps[j] : t;
        if (pj == vpos && t - pj >= P.recent) s_victim = j;  // positions are distinct
      }
    }
    __syncthreads();
    victim = s_victim;
  }
  // 6. writes
  if (append) {
    // ranks: cached positions above the new one move up by one
    for (int j = tid; j < n; j += kThreads)
      if (rk[j] >= new_rank) rk[j] = rk[j] + 1;
    if (tid == 0) {
      rk[n] = new_rank;
      ps[n] = t;
      P.seq_len[u] = n + 1;
      P.evicted[u] = -1;
    }
    for (int q = tid; q < W; q += kThreads) hs[(size_t)q * ms + n] = 0.f;
    if (tid < LPT) {
      const size_t row = ((size_t)s_blk * kBlock + n % kBlock) * row_bytes + tid * 16;
      st16(P.k_pool + row, ld16(P.k_new + (size_t)u * row_bytes + tid * 16));
      st16(P.v_pool + row, ld16(P.v_new + (size_t)u * row_bytes + tid * 16));
    }
    return;
  }
  if (victim < 0 || victim == n) {  // no candidate, or the new token itself is dropped
    if (tid == 0) P.evicted[u] = t;
    return;
  }
  const int cr_v = rk[victim] + (rk[victim] >= new_rank ? 1 : 0);
  const int vpos = ps[victim];
  __syncthreads();  // every thread has read the victim's rank and position
  for (int j = tid; j < n; j += kThreads) {
    if (j == victim) continue;
    const int cr = rk[j] + (rk[j] >= new_rank ? 1 : 0);
    rk[j] = cr - (cr > cr_v ? 1 : 0);
  }
  if (tid == 0) {
    rk[victim] = new_rank - (new_rank > cr_v ? 1 : 0);
    ps[victim] = t;
    P.evicted[u] = vpos;
  }
  for (int q = tid; q < W; q += kThreads) hs[(size_t)q * ms + victim] = 0.f;
  if (tid < LPT) {
    const size_t row =
        ((size_t)s_bt[victim / kBlock] * kBlock + victim % kBlock) * row_bytes + tid * 16;
    st16(P.k_pool + row, ld16(P.k_new + (size_t)u * row_bytes + tid * 16));
    st16(P.v_pool + row, ld16(P.v_new + (size_t)u * row_bytes + tid * 16));
  }
}

// The ring state of a cache: zero rings, index 0, and each slot's index in
// position order (a count over the head's positions, staged in LDS).
__global__ __launch_bounds__(kThreads) void ring_init_kernel(const RingArgs P) {
  __shared__ int s_pos[kRingMaxBudget];
  const int u = blockIdx.x, tid = threadIdx.x, ms = P.max_slots;
  float *hs = P.hist + (size_t)u * P.W * ms;
  for (size_t i = tid; i < (size_t)P.W * ms; i += kThreads) hs[i] = 0.f;
  if (tid == 0) P.ring[u] = 0;
  const int n = P.seq_len[u];
  if (n < 0 || n > kRingMaxBudget || n > ms) return;  // refused by the step as well
  const int32_t *ps = P.pos + (size_t)u * ms;
  for (int j = tid; j < n; j += kThreads) s_pos[j] = ps[j];
  __syncthreads();
  for (int j = tid; j < n; j += kThreads) {
    const int pj = s_pos[j];
    int c = 0;
    for (int i = 0; i < n; ++i) c += s_pos[i] < pj ? 1 : 0;
    P.rank[(size_t)u * ms + j] = c;
  }
}

hipError_t launch_ring_init(const RingArgs &a, hipStream_t s) {
  if (a.units == 0) return hipSuccess;
  hipLaunchKernelGGL(ring_init_kernel, dim3((unsigned)a.units), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

size_t ring_lds_bytes(const RingArgs &a) { return ((size_t)a.G * (a.budget + 1) + a.budget + 1) * 4; }

template <bool BF16, int LPT>
static hipError_t launch_t(const RingArgs &a, hipStream_t s) {
  auto fn = ring_step_kernel<BF16, LPT>;
  const size_t lds = ring_lds_bytes(a);
  if (lds > 65536) {  // idempotent: set on every such launch, no cached state
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(fn),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(fn, dim3((unsigned)a.units), dim3(kThreads), lds, s, a);
  return hipGetLastError();
}

hipError_t launch_ring_step(const RingArgs &a, int bf16, int head_dim, hipStream_t s) {
  if (a.units == 0) return hipSuccess;
  if (bf16) return head_dim == 128 ? launch_t<true, 16>(a, s) : launch_t<true, 8>(a, s);
  return head_dim == 128 ? launch_t<false, 32>(a, s) : launch_t<false, 16>(a, s);
}

}  // namespace kvev
