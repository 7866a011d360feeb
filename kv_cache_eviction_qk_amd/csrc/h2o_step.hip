// h2o_step.hip -- one H2O decode step of every KV head (gfx950).
//
// [H2O] "Step-by-Step Eviction Lifecycle": the new token's query rows (the G
// query heads of the KV head) attend to the cached tokens and to the token
// itself; the weights, summed over the G rows, join each token's running
// score; at the budget the token with the smallest (score, position) outside
// the recent window is pruned, and the new token overwrites its slot in place
// ([H2O] "PagedAttention Memory Integration").  Below the budget the token is
// appended, taking a block from the free list when its logical block has none.
//
// One 1024-thread workgroup per KV head, one launch per step:
//   1. block ids of the head to LDS (checked), the running scores and
//      positions of the thread's slots, the new K / V row: one round of loads;
//   2. logits: the G query rows (padded to 16) against 16 keys per MFMA
//      (v_mfma 16x16, bf16 or fp32), each wave a strided set of blocks with
//      up to 16 / U blocks in flight; the new key by one wave; log2 units
//      into LDS;
//   3. per query row (one wave each) the log-sum-exp over the cached tokens
//      and the new one;
//   4. p = exp2(logit - lse) summed over the rows in order and added to the
//      thread's scores; the candidates' (score key, position) packed into 64
//      bits, the workgroup minimum found by wave shuffles;
//   5. writes: every score once, the new token's K / V row, position and
//      score at the pruned slot (or slot n), seq_len on append.
// Every global address is written by one thread of one workgroup, so no
// cross-workgroup ordering is involved; the free list is the only shared
// state (one atomic per head that appends into a fresh block).
#include <hip/hip_runtime.h>

#include "kvev_device.h"
#include "kvev_kernels.h"

namespace kvev {

namespace {
constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / kWave;             // 16
constexpr int kPer = kH2oMaxBudget / kThreads;       // slots per thread (4)
constexpr int kMaxBlocksH = kH2oMaxBudget / kBlock;  // 256

__device__ __forceinline__ unsigned long long pack_min(float v, int p) {
  // (score key, position) ordered as one unsigned word; the sign flip keeps
  // signed positions in order
  return ((unsigned long long)score_key(v) << 32) | (unsigned long long)((uint32_t)p ^ 0x80000000u);
}

__device__ __forceinline__ unsigned long long wave_min_u64(unsigned long long v) {
#pragma unroll
  for (int o = kWave / 2; o >= 1; o >>= 1) {
    const uint32_t lo = __shfl_xor((uint32_t)v, o), hi = __shfl_xor((uint32_t)(v >> 32), o);
    const unsigned long long w = ((unsigned long long)hi << 32) | lo;
    v = w < v ? w : v;
  }
  return v;
}
}  // namespace

template <bool BF16, int D>
__global__ __launch_bounds__(kThreads) void h2o_step_kernel(const H2oArgs P) {
  constexpr int EB = BF16 ? 2 : 4, ROWB = D * EB, U = ROWB / 64, CPR = ROWB / 16;
  constexpr int NBK = (16 / U) > 0 ? 16 / U : 1;  // blocks per load batch of a wave
  extern __shared__ float lgt[];                  // [G][np] logits, log2 units
  __shared__ int s_bt[kMaxBlocksH + 1];
  __shared__ unsigned long long s_wmin[kWaves];
  __shared__ float s_lse[16], s_newlg[16];
  __shared__ float s_snew;
  __shared__ int s_bad, s_dst, s_fresh;

  const int u = blockIdx.x, tid = threadIdx.x, l = lane_id(), lr = l & 15, lg = l >> 4;
  const int wv = tid / kWave;
  const int b = u / P.Hkv, h = u % P.Hkv;
  const int G = P.G, budget = P.budget, NP = P.np;
  int32_t *bt = P.block_table + (size_t)u * P.max_blocks;
  int32_t *ps = P.pos + (size_t)u * P.max_slots;
  float *sc = P.score + (size_t)u * P.max_slots;

  // ---- one round of loads: length, position, block ids, scores, the new row
  const int n = P.seq_len[u];
  const int t = P.t_pos[b];
  if (n < 0 || n > budget) {  // inconsistent head: left unchanged
    if (tid == 0) P.evicted[u] = -2;
    return;
  }
  const bool append = n < budget;
  const int nb = (n + kBlock - 1) / kBlock;      // blocks holding cached tokens
  const int nbt = append ? n / kBlock + 1 : nb;  // entries the step touches
  const int my_id = tid < nbt ? bt[tid] : 0;     // nbt <= 257 <= kThreads
  float scv[kPer];
  int psv[kPer];
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int j = tid + k * kThreads;
    scv[k] = j < n ? sc[j] : 0.f;
    psv[k] = j < n ? ps[j] : 0;
  }
  // the new K / V row: lanes 0..CPR-1 of wave 0 hold K pieces, 32..32+CPR-1 V
  uint4 newrow = make_uint4(0u, 0u, 0u, 0u);
  if (wv == 0 && (l & 31) < CPR)
    newrow = ld16((l < 32 ? P.k_new : P.v_new) + (size_t)u * ROWB + (size_t)(l & 31) * 16);
  if (tid == 0) {
    s_bad = 0;
    s_fresh = -1;
  }
  __syncthreads();
  if (tid < nbt) {
    // the append slot's entry may be -1: a block is taken from the free list
    const bool fresh_ok = append && tid == n / kBlock && n % kBlock == 0 && my_id < 0;
    if (!fresh_ok && (my_id < 0 || my_id >= P.num_blocks)) s_bad = 1;
    s_bt[tid] = my_id;
  }
  __syncthreads();
  if (s_bad) {
    if (tid == 0) P.evicted[u] = -4;
    return;
  }
  if (tid == 0 && append && n % kBlock == 0 && s_bt[n / kBlock] < 0) {
    const int old = atomicSub(P.free_count, 1);
    int code = 0;
    if (old <= 0) {
      atomicAdd(P.free_count, 1);
      code = -3;
    } else {
      const int blk = P.free_list[old - 1];
      if (blk < 0 || blk >= P.num_blocks) code = -4;  // a bad entry stays taken
      else {
        s_bt[n / kBlock] = blk;
        bt[n / kBlock] = blk;
      }
    }
    s_fresh = code;
  }
  __syncthreads();
  if (s_fresh < -1) {
    if (tid == 0) P.evicted[u] = s_fresh;
    return;
  }

  // ---- logits of the G query rows (rows past G repeat the last one and are
  // not stored): A = query rows, B = 16 keys of a block
  const int Hq = P.Hkv * G;
  const uint8_t *qbase = P.q + ((size_t)b * Hq + (size_t)h * G + min(lr, G - 1)) * ROWB;
  uint4 qa[U];
#pragma unroll
  for (int j = 0; j < U; ++j) qa[j] = ld16(qbase + (lg * U + j) * 16);
  const float c1 = P.c1;
  const size_t lane_off = (size_t)lr * ROWB + (size_t)lg * (ROWB / 4);
  if (wv == kWaves - 1) {
    // the new key against every row: all 16 B columns are the same key
    uint4 kn[U];
#pragma unroll
    for (int j = 0; j < U; ++j) kn[j] = ld16(P.k_new + (size_t)u * ROWB + lg * (ROWB / 4) + 16 * j);
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < U; ++j) acc = mfma_unit<BF16>(qa[j], kn[j], acc);
    if (lr == 0) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (4 * lg + e < G) s_newlg[4 * lg + e] = acc[e] * c1;
    }
  }
  for (int lb0 = wv; lb0 < nb; lb0 += kWaves * NBK) {  // wave-uniform
    uint4 kf[NBK][U];
    int kp[NBK];
#pragma unroll
    for (int i = 0; i < NBK; ++i) {
      const int lb = min(lb0 + i * kWaves, nb - 1);
      const uint8_t *src = P.k_pool + (size_t)s_bt[lb] * kBlock * ROWB + lane_off;
#pragma unroll
      for (int j = 0; j < U; ++j) kf[i][j] = ld16(src + 16 * j);
      kp[i] = ps[lb * kBlock + lr];
    }
#pragma unroll
    for (int i = 0; i < NBK; ++i) {
      const int lb = lb0 + i * kWaves;
      if (lb >= nb) break;
      floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < U; ++j) acc = mfma_unit<BF16>(qa[j], kf[i][j], acc);
      const int slot = lb * kBlock + lr;
      const bool live = slot < n && kp[i] <= t;  // later positions are not attended
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (4 * lg + e < G) lgt[(4 * lg + e) * NP + slot] = live ? acc[e] * c1 : -__builtin_inff();
    }
  }
  __syncthreads();

  // ---- log-sum-exp of each query row (log2 units), one wave per row
  for (int g = wv; g < G; g += kWaves) {
    const float *row = lgt + (size_t)g * NP;
    float mx = s_newlg[g];
    for (int j = l; j < n; j += kWave) mx = fmaxf(mx, row[j]);
#pragma unroll
    for (int o = kWave / 2; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
    float z = 0.f;
    for (int j = l; j < n; j += kWave) z += __builtin_amdgcn_exp2f(row[j] - mx);
#pragma unroll
    for (int o = kWave / 2; o >= 1; o >>= 1) z += __shfl_xor(z, o);
    z += __builtin_amdgcn_exp2f(s_newlg[g] - mx);
    if (l == 0) s_lse[g] = mx + __builtin_amdgcn_logf(z);
  }
  __syncthreads();

  // ---- running scores, the new token's score, the candidates' minimum
  unsigned long long best = ~0ull;
  const long long R = P.recent;
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int j = tid + k * kThreads;
    if (j < n) {
      float p = 0.f;
      for (int g = 0; g < G; ++g) p += __builtin_amdgcn_exp2f(lgt[(size_t)g * NP + j] - s_lse[g]);
      scv[k] += p;
      if ((long long)t - psv[k] >= R) {
        const unsigned long long c = pack_min(scv[k], psv[k]);
        best = c < best ? c : best;
      }
    }
  }
  float snew = 0.f;
  if (tid == 0) {
    for (int g = 0; g < G; ++g) snew += __builtin_amdgcn_exp2f(s_newlg[g] - s_lse[g]);
    s_snew = snew;
    if (R == 0) {  // the new token competes too
      const unsigned long long c = pack_min(snew, t);
      best = c < best ? c : best;
    }
    s_dst = append ? n : -1;  // -1: the new token is dropped unless a slot wins
  }
  best = wave_min_u64(best);
  if (l == 0) s_wmin[wv] = best;
  __syncthreads();
  unsigned long long m = s_wmin[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) m = s_wmin[w] < m ? s_wmin[w] : m;
  int victim_k = -1;  // which of this thread's slots is pruned
  if (!append && m != ~0ull) {
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int j = tid + k * kThreads;
      if (j < n && (long long)t - psv[k] >= R && pack_min(scv[k], psv[k]) == m) {
        victim_k = k;
        s_dst = j;
      }
    }
  }
  __syncthreads();

  // ---- writes: each score once; the new token at slot dst
  const int dst = s_dst;
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int j = tid + k * kThreads;
    if (j < n && j != dst) sc[j] = scv[k];
  }
  if (victim_k >= 0) P.evicted[u] = psv[victim_k];
  if (tid == 0) {
    if (append) {
      P.evicted[u] = -1;
      P.seq_len[u] = n + 1;
    } else if (dst < 0) {
      P.evicted[u] = t;
    }
    if (dst >= 0) {
      sc[dst] = s_snew;
      ps[dst] = t;
    }
  }
  if (wv == 0 && dst >= 0 && (l & 31) < CPR) {
    const size_t row = (size_t)s_bt[dst / kBlock] * kBlock + dst % kBlock;
    st16((l < 32 ? P.k_pool : P.v_pool) + row * ROWB + (size_t)(l & 31) * 16, newrow);
  }
}

hipError_t launch_h2o_step(const H2oArgs &a, int bf16, int head_dim, hipStream_t s) {
  const size_t lds = (size_t)a.G * a.np * sizeof(float);
  const dim3 grid((unsigned)a.units), block(kThreads);
  if (bf16) {
    if (head_dim == 128) hipLaunchKernelGGL((h2o_step_kernel<true, 128>), grid, block, lds, s, a);
    else hipLaunchKernelGGL((h2o_step_kernel<true, 64>), grid, block, lds, s, a);
  } else {
    if (head_dim == 128) hipLaunchKernelGGL((h2o_step_kernel<false, 128>), grid, block, lds, s, a);
    else hipLaunchKernelGGL((h2o_step_kernel<false, 64>), grid, block, lds, s, a);
  }
  return hipGetLastError();
}

}  // namespace kvev
