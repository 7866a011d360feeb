// ring_step.hip -- one decode step of SnapKV's ring-buffer adaptation for
// every KV head (gfx950).
//
// [SNAP] "How it works" and "On the adaptation": each cached token keeps a
// ring of its last obsWindow observed attention weights; an observed step
// writes every cached token's weight at the ring index and advances it (a
// null step writes nothing and does not advance); the new token enters with
// a zero ring; over the budget, the ring sums are max-pooled over the
// poolKernel tokens centred on each in position order (clamped) and the
// smallest (pooled, position) outside the recent window is dropped, equal
// scores dropping the lower position.
//
// One launch per step; each KV head is split over `split` 1024-thread
// workgroups, each taking a contiguous range of the budget's blocks (a range
// of the budget, not of the head's length, so that the block ids load in
// the same round as the length):
//   part  (every workgroup of the head): logits of the G query rows (padded
//         to 16) against 16 keys per MFMA, in log2 units; the part's
//         maximum m and sum l = sum exp2(logit - m) per row (part 0 also
//         counts the new token) and e = exp2(logit - m) of its slots; at the
//         budget, for each of its slots the sum of the ring entries other
//         than the one this step writes (index order).  All of it goes to
//         the workspace with agent-scope atomic stores; once they have
//         completed, one agent-scope atomic on the head's arrival counter.
//   final (the workgroup that arrives last): the checks (block ids, ranks);
//         lse of each row from the parts' (m, l) in order; each cached
//         slot's weight, the sum over the rows (ascending) of
//         e * exp2(m - lse), written at the ring index; at the budget the
//         ring sum (the other entries' sum plus the weight), laid out in
//         position order through the persistent ranks, the pooled maximum
//         and the packed (score key, position) minimum over the candidates;
//         then every write of the step: ranks, the new token's K/V row,
//         position and zero ring, seq_len, the ring index, the arrival
//         counter reset.
// Ranks make position order available without a sort: they are kept as each
// slot's index in position order and updated in one parallel pass.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "kvev_device.h"
#include "kvev_kernels.h"

namespace kvev {

namespace {
constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / kWave;          // 16
constexpr int kMaxSplit = kRingMaxSplit;
constexpr int kHB = 16;                           // ring entries of a slot per thread in flight

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
// ---- agent-scope accesses for data another workgroup of the launch reads
__device__ __forceinline__ void cst(uint32_t *p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t cld(const uint32_t *p) {
  return __hip_atomic_load(const_cast<uint32_t *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// every memory operation this wave issued has completed
__device__ __forceinline__ void drain() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}
}  // namespace

// G <= kRingMaxGroup; D = 64 or 128; kPer slots per thread in the final
// step: budget <= kPer * 1024 (1 up to 1024 tokens, which keeps the final
// step's code short, else 4).
template <bool BF16, int D, int kPer>
__global__ __launch_bounds__(kThreads) void ring_step_kernel(const RingArgs P) {
  constexpr int EB = BF16 ? 2 : 4, ROWB = D * EB, U = ROWB / 64, CPR = ROWB / 16;
  constexpr int NBK = U >= 8 ? 1 : 8 / U;  // blocks per load batch of a wave
  extern __shared__ float lds[];  // part: logits [G][cb*16]; final: ring sums in position order
  __shared__ int s_bt[kRingMaxBlocks];
  __shared__ float s_newlg[16], s_m[16], s_l[16];
  __shared__ __align__(16) float s_r[kMaxSplit][kRingMaxGroup];  // exp2(m - lse), part-major
  __shared__ unsigned long long s_wmin[kWaves];
  __shared__ int s_cnt[kWaves];
  __shared__ int s_last, s_code, s_blk, s_pop, s_bad, s_dst, s_crv, s_vpos;

  const int S = P.split;
  const int u = blockIdx.x / S, w = blockIdx.x % S;
  const int tid = threadIdx.x, l = lane_id(), lr = l & 15, lg = l >> 4, wv = tid / kWave;
  const int b = u / P.Hkv, h = u % P.Hkv;
  const int G = P.G, W = P.W, ms = P.max_slots, budget = P.budget, np = P.np;
  int32_t *bt = P.block_table + (size_t)u * P.max_blocks;
  int32_t *ps = P.pos + (size_t)u * ms;
  int32_t *rk = P.rank + (size_t)u * ms;
  float *hs = P.hist + (size_t)u * W * ms;
  uint32_t *E = P.e + (size_t)u * G * np;             // [G][np]: e of every slot
  uint32_t *RS = P.rsum + (size_t)u * np;             // the other ring entries' sum of every slot
  uint32_t *ML = P.ml + (size_t)u * kMaxSplit * 32;   // [split][16 m, 16 l]

  // ---------------------------------------------------------------- part
  // one round of loads, none waiting for another: the head's state, every
  // block id of the budget (the part uses its range; the final step checks
  // them all and needs the victim's), the query rows, and what the final
  // step needs, loaded by every part so that the one arriving last has it
  // at hand (the positions and ranks of the thread's slots, the new K / V
  // row: lanes 0..CPR-1 of wave 0 hold K pieces, 32..32+CPR-1 V)
  const int n = P.seq_len[u];
  const int t = P.t_pos[b];
  const int ring0 = P.ring[u];
  const bool observe = P.observe[b] != 0;
  const int all_id = tid < P.nbmax ? bt[tid] : 0;
  const int Hq = P.Hkv * G;
  const uint8_t *qbase = P.q + ((size_t)b * Hq + (size_t)h * G + min(lr, G - 1)) * ROWB;
  uint4 qa[U];
#pragma unroll
  for (int j = 0; j < U; ++j) qa[j] = ld16(qbase + (lg * U + j) * 16);
  int psv[kPer], rkv[kPer];
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int j = tid + k * kThreads;
    psv[k] = j < budget ? ps[j] : 0;
    rkv[k] = j < budget ? rk[j] : 0;
  }
  uint4 newrow = make_uint4(0u, 0u, 0u, 0u);
  if (wv == 0 && (l & 31) < CPR)
    newrow = ld16((l < 32 ? P.k_new : P.v_new) + (size_t)u * ROWB + (size_t)(l & 31) * 16);
  if (n < 0 || n > budget || ring0 < 0 || ring0 >= W) {
    // inconsistent head: left unchanged, no part arrives
    if (w == 0 && tid == 0) P.evicted[u] = -2;
    return;
  }
  const bool append = n < budget;
  const int nb = (n + kBlock - 1) / kBlock;  // blocks holding cached tokens
  const int cb = P.cb;
  const int lb0 = w * cb, lb1 = min(lb0 + cb, nb);
  const int pnb = max(0, lb1 - lb0);          // the part's blocks holding cached tokens
  const int ps0 = lb0 * kBlock, pslots = max(0, min(lb1 * kBlock, n) - ps0);
  const int CS = cb * kBlock;                 // LDS row stride of the logits
  if (tid == 0) s_bad = 0;
  // block ids; a bad one reads block 0 here and is refused by the final step
  if (tid < nb) s_bt[tid] = (all_id < 0 || all_id >= P.num_blocks) ? 0 : all_id;
  __syncthreads();
  if (tid < nb && (all_id < 0 || all_id >= P.num_blocks)) s_bad = 1;
  // at the budget: the first ring entries of the part's first slots, in
  // flight with the keys (two threads a slot, kHB entries each)
  const int hj = tid >> 1, hh = tid & 1;
  float hr[kHB];
#pragma unroll
  for (int i = 0; i < kHB; ++i) hr[i] = 0.f;
  if (!append && hj < pslots) {
#pragma unroll
    for (int i = 0; i < kHB; ++i) hr[i] = hs[(size_t)min(hh * kHB + i, W - 1) * ms + ps0 + hj];
  }

  const float c1 = P.c1;
  const size_t lane_off = (size_t)lr * ROWB + (size_t)lg * (ROWB / 4);
  // the part's blocks, and in part 0 one more: the new key against every
  // row (all 16 columns the same key)
  const int vnb = pnb + (w == 0 ? 1 : 0);
  for (int ib = wv; ib < vnb; ib += kWaves * NBK) {  // wave-uniform
    uint4 kf[NBK][U];
    int kp[NBK];
    // branch-free, so that every load of the batch is in flight at once:
    // past the last block a repeat of it (or of the new key), not used
#pragma unroll
    for (int i = 0; i < NBK; ++i) {
      const int lb = ib + i * kWaves;
      const int lbc = min(lb, max(pnb - 1, 0));
      const uint8_t *src = lb >= pnb ? P.k_new + (size_t)u * ROWB + (size_t)lg * (ROWB / 4)
                                     : P.k_pool + (size_t)s_bt[lb0 + lbc] * kBlock * ROWB + lane_off;
#pragma unroll
      for (int j = 0; j < U; ++j) kf[i][j] = ld16(src + 16 * j);
      kp[i] = ps[(lb0 + lbc) * kBlock + lr];
    }
#pragma unroll
    for (int i = 0; i < NBK; ++i) {
      const int lb = ib + i * kWaves;
      if (lb >= vnb) break;
      floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < U; ++j) acc = mfma_unit<BF16>(qa[j], kf[i][j], acc);
      if (lb == pnb) {  // the new key
        if (lr == 0) {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (4 * lg + e < G) s_newlg[4 * lg + e] = acc[e] * c1;
        }
        continue;
      }
      const int slot = (lb0 + lb) * kBlock + lr;
      const bool live = slot < n && kp[i] <= t;  // later positions are not attended
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (4 * lg + e < G) lds[(4 * lg + e) * CS + lb * kBlock + lr] = live ? acc[e] * c1 : -__builtin_inff();
    }
  }
  __syncthreads();
  // the part's maximum and sum per row (one wave per row)
  for (int g = wv; g < G; g += kWaves) {
    const float *row = lds + (size_t)g * CS;
    float mx = w == 0 ? s_newlg[g] : -__builtin_inff();
    for (int j = l; j < pslots; j += kWave) mx = fmaxf(mx, row[j]);
#pragma unroll
    for (int o = kWave / 2; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
    float z = 0.f;
    if (mx != -__builtin_inff()) {  // a part whose keys are all masked holds no weight
      for (int j = l; j < pslots; j += kWave) z += __builtin_amdgcn_exp2f(row[j] - mx);
    }
#pragma unroll
    for (int o = kWave / 2; o >= 1; o >>= 1) z += __shfl_xor(z, o);
    if (w == 0) z += __builtin_amdgcn_exp2f(s_newlg[g] - mx);  // mx is finite in part 0
    if (l == 0) {
      s_m[g] = mx;
      s_l[g] = z;
    }
  }
  // at the budget: the ring entries of each slot other than the one this
  // step writes, summed in index order (the final step adds the weight).
  // Two adjacent lanes share a slot: of each 2 * kHB entries the even lane
  // holds the first kHB, the odd lane the rest; the even lane's running sum
  // passes to the odd lane, which continues it, and back.  Into LDS, after
  // the logits.
  float *rsl = lds + (size_t)G * CS;
  if (!append) {
    for (int jl0 = 0; jl0 < pslots; jl0 += kThreads / 2) {  // uniform
      const int jl = jl0 + hj;
      const int j = ps0 + min(jl, pslots - 1);
      float acc = 0.f;
      for (int q0 = 0; q0 < W; q0 += 2 * kHB) {
        float hv[kHB];
        if (q0 == 0 && jl0 == 0) {
#pragma unroll
          for (int i = 0; i < kHB; ++i) hv[i] = hr[i];
        } else {
#pragma unroll
          for (int i = 0; i < kHB; ++i) hv[i] = hs[(size_t)min(q0 + hh * kHB + i, W - 1) * ms + j];
        }
        auto run = [&](float c) {
#pragma unroll
          for (int i = 0; i < kHB; ++i) {
            const int q = q0 + hh * kHB + i;
            c += (q < W && !(observe && q == ring0)) ? hv[i] : 0.f;
          }
          return c;
        };
        const float even = run(acc);                   // meaningful in the even lane
        const float odd = run(__shfl_xor(even, 1));    // meaningful in the odd lane
        acc = __shfl(odd, l | 1);
      }
      if (hh == 0 && jl < pslots) rsl[jl] = acc;
    }
  }
  __syncthreads();
  // publication, every store of the part after its last barrier before the
  // arrival (a workgroup barrier waits for the stores issued before it)
  for (int i = tid; i < G * pslots; i += kThreads) {
    const int g = i / pslots, j = i % pslots;
    const float m = s_m[g];
    const float e = m == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(lds[(size_t)g * CS + j] - m);
    cst(E + (size_t)g * np + ps0 + j, __float_as_uint(e));
  }
  if (!append)
    for (int j = tid; j < pslots; j += kThreads) cst(RS + ps0 + j, __float_as_uint(rsl[j]));
  if (tid < G) {
    cst(ML + w * 32 + tid, __float_as_uint(s_m[tid]));
    cst(ML + w * 32 + 16 + tid, __float_as_uint(s_l[tid]));
  }
  // Hand-off: every value another workgroup reads is written and read with
  // agent-scope atomics (stores through to the agent's coherence point,
  // loads from it), and each wave waits for its stores to complete before
  // the barrier that precedes the arrival; the last part's loads are issued
  // after its arrival returned.  A release/acquire arrival would add the L2
  // write-back and invalidate that plain (non-atomic) data needs; nothing
  // here hands over plain data.
  drain();
  __syncthreads();
  if (tid == 0)
    s_last = __hip_atomic_fetch_add(P.arrive + u, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
             (uint32_t)(S - 1);
  __syncthreads();
  if (!s_last) return;

  // --------------------------------------------------------------- final
  // one round of loads: the e values and ring sums of the thread's slots,
  // every part's (m, l)
  float ev[kPer][kRingMaxGroup], rv[kPer];
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int j = tid + k * kThreads;
#pragma unroll
    for (int g = 0; g < kRingMaxGroup; ++g)
      ev[k][g] = (j < n && g < G) ? __uint_as_float(cld(E + (size_t)g * np + j)) : 0.f;
    rv[k] = (!append && j < n) ? __uint_as_float(cld(RS + j)) : 0.f;
  }
  float mq[kMaxSplit], lq[kMaxSplit];
#pragma unroll
  for (int q = 0; q < kMaxSplit; ++q) {
    mq[q] = -__builtin_inff();
    lq[q] = 0.f;
  }
  if (tid < G) {
#pragma unroll
    for (int q = 0; q < kMaxSplit; ++q) {
      mq[q] = q < S ? __uint_as_float(cld(ML + q * 32 + tid)) : -__builtin_inff();
      lq[q] = q < S ? __uint_as_float(cld(ML + q * 32 + 16 + tid)) : 0.f;
    }
  }
  // ranks outside [0, n) (not left by the ring step or its init): refused;
  // the cached positions below the new one (its rank), counted per wave
  int below = 0;
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int j = tid + k * kThreads;
    if (j < n && (unsigned)rkv[k] >= (unsigned)n) s_bad = 2;
    below += __popcll(__ballot(j < n && psv[k] < t));
  }
  if (l == 0) s_cnt[wv] = below;
  // lse of each row from the parts' (m, l), parts in order; r = exp2(m - lse)
  // (0 for the rows past G)
  if (tid < kRingMaxGroup) {
    float M = -__builtin_inff();
#pragma unroll
    for (int q = 0; q < kMaxSplit; ++q) M = fmaxf(M, mq[q]);
    float Z = 0.f;
#pragma unroll
    for (int q = 0; q < kMaxSplit; ++q)
      if (mq[q] != -__builtin_inff()) Z += lq[q] * __builtin_amdgcn_exp2f(mq[q] - M);
    const float lse = M + __builtin_amdgcn_logf(Z);
#pragma unroll
    for (int q = 0; q < kMaxSplit; ++q)
      s_r[q][tid] = mq[q] == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(mq[q] - lse);
  }
  __syncthreads();
  // (stores here would hold up the barriers that follow: the arrival
  // counter, the ring index and a new block's table entry are written last)
  if (tid == 0) {
    int code = s_bad == 2 ? -2 : s_bad ? -4 : 0, blk = -1, pop = 0;
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
          else pop = 1;
        }
      }
    }
    s_code = code;
    s_blk = blk;
    s_pop = pop;
    s_dst = -1;
  }
  __syncthreads();
  if (s_code) {
    if (tid == 0) {
      cst(P.arrive + u, 0u);  // state for the next call
      P.evicted[u] = s_code;
    }
    return;
  }
  int new_rank = 0;
#pragma unroll
  for (int q = 0; q < kWaves; ++q) new_rank += s_cnt[q];

  // each cached slot's weight (rows ascending; the rows past G add 0 * 0)
  // and, at the budget, its ring sum
  float wk[kPer], sv[kPer];
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int j = tid + k * kThreads;
    const int q = min((j / kBlock) / P.cb, kMaxSplit - 1);
    const float4 r0 = *reinterpret_cast<const float4 *>(&s_r[q][0]);
    const float4 r1 = *reinterpret_cast<const float4 *>(&s_r[q][4]);
    const float rr[kRingMaxGroup] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w};
    float p = 0.f;
#pragma unroll
    for (int g = 0; g < kRingMaxGroup; ++g) p += ev[k][g] * rr[g];
    wk[k] = p;
    sv[k] = observe ? rv[k] + p : rv[k];
  }

  // at the budget: position-ordered sums, pooling, the victim
  int victim = -1;  // slot, n for the new token
  if (!append) {
    float *ord = lds;  // [n + 1], over the part's logits (no longer read)
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int j = tid + k * kThreads;
      if (j < n) ord[rkv[k] + (rkv[k] >= new_rank ? 1 : 0)] = sv[k];
    }
    if (tid == 0) ord[new_rank] = 0.f;
    __syncthreads();
    const int r = (P.pool_kernel - 1) / 2;
    const long long R = P.recent;
    // the maximum over [cr - r, cr + r] clamped to [0, n]: small windows as
    // one batch of reads (clamped indices repeat an end, which leaves the
    // maximum unchanged), larger ones in order
    auto pooled = [&](int cr) {
      const int lo = max(0, cr - r), hi = min(n, cr + r);
      float m = ord[lo];
      if (r <= 3) {
#pragma unroll
        for (int i = -3; i <= 3; ++i) m = fmaxf(m, ord[min(max(cr + i, lo), hi)]);
      } else if (r <= 8) {
#pragma unroll
        for (int i = -8; i <= 8; ++i) m = fmaxf(m, ord[min(max(cr + i, lo), hi)]);
      } else {
        for (int i = lo + 1; i <= hi; ++i) m = fmaxf(m, ord[i]);
      }
      return m;
    };
    unsigned long long best = ~0ull, key[kPer], knew = ~0ull;
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int j = tid + k * kThreads;
      key[k] = ~0ull;
      if (j < n && (long long)t - psv[k] >= R) {
        key[k] = pack_min(pooled(rkv[k] + (rkv[k] >= new_rank ? 1 : 0)), psv[k]);
        best = key[k] < best ? key[k] : best;
      }
    }
    if (tid == 0 && R == 0) {  // the new token competes too
      knew = pack_min(pooled(new_rank), t);
      best = knew < best ? knew : best;
    }
    best = wave_min_u64(best);
    if (l == 0) s_wmin[wv] = best;
    __syncthreads();
    unsigned long long mn = s_wmin[0];
#pragma unroll
    for (int q = 1; q < kWaves; ++q) mn = s_wmin[q] < mn ? s_wmin[q] : mn;
    if (mn != ~0ull) {  // positions are distinct: one slot (or the new token) holds the minimum
#pragma unroll
      for (int k = 0; k < kPer; ++k) {
        if (key[k] == mn) {
          s_dst = tid + k * kThreads;
          s_crv = rkv[k] + (rkv[k] >= new_rank ? 1 : 0);
          s_vpos = psv[k];
        }
      }
      if (knew == mn) s_dst = n;
    }
    __syncthreads();
    victim = s_dst;
  }

  // writes: the state (arrival counter, ring index, a new block's table
  // entry), the weights at the ring index (a zero ring for the slot the new
  // token takes), the ranks, the new token
  if (tid == 0) {
    cst(P.arrive + u, 0u);  // state for the next call
    if (observe) P.ring[u] = ring0 + 1 == W ? 0 : ring0 + 1;
    if (s_pop) bt[n / kBlock] = s_blk;
  }
  const int dst = append ? n : (victim >= 0 && victim < n ? victim : -1);
  if (observe) {
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int j = tid + k * kThreads;
      if (j < n) hs[(size_t)ring0 * ms + j] = j == dst ? 0.f : wk[k];
    }
  }
  if (dst >= 0) {
    for (int q = tid; q < W; q += kThreads)
      if (!(observe && q == ring0 && dst < n)) hs[(size_t)q * ms + dst] = 0.f;
  }
  if (append) {
    // ranks: cached positions above the new one move up by one
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int j = tid + k * kThreads;
      if (j < n && rkv[k] >= new_rank) rk[j] = rkv[k] + 1;
    }
    if (tid == 0) {
      rk[n] = new_rank;
      ps[n] = t;
      P.seq_len[u] = n + 1;
      P.evicted[u] = -1;
    }
  } else if (dst < 0) {  // no candidate, or the new token itself is dropped
    if (tid == 0) P.evicted[u] = t;
    return;
  } else {
    const int cr_v = s_crv;
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int j = tid + k * kThreads;
      if (j < n && j != dst) {
        const int cr = rkv[k] + (rkv[k] >= new_rank ? 1 : 0);
        const int nr = cr - (cr > cr_v ? 1 : 0);
        if (nr != rkv[k]) rk[j] = nr;
      }
    }
    if (tid == 0) {
      rk[dst] = new_rank - (new_rank > cr_v ? 1 : 0);
      ps[dst] = t;
      P.evicted[u] = s_vpos;
    }
  }
  if (wv == 0 && (l & 31) < CPR) {
    const int blk = append ? s_blk : s_bt[dst / kBlock];
    const size_t row = (size_t)blk * kBlock + dst % kBlock;
    st16((l < 32 ? P.k_pool : P.v_pool) + row * ROWB + (size_t)(l & 31) * 16, newrow);
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

size_t ring_lds_bytes(const RingArgs &a) {
  // a part's logits ([G][cb*16]) and ring sums ([cb*16]), or the final
  // step's position-ordered sums ([budget + 1])
  return std::max((size_t)(a.G + 1) * a.cb * kBlock, (size_t)a.budget + 1) * sizeof(float);
}

template <bool BF16, int D>
static hipError_t launch_t(const RingArgs &a, hipStream_t s) {
  static_assert(4 * kThreads >= kRingMaxBudget, "the final step covers the budget");
  auto fn = a.budget <= kThreads ? ring_step_kernel<BF16, D, 1> : ring_step_kernel<BF16, D, 4>;
  const size_t lds = ring_lds_bytes(a);
  if (lds > 65536) {  // idempotent: set on every such launch, no cached state
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(fn),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(fn, dim3((unsigned)(a.units * a.split)), dim3(kThreads), lds, s, a);
  return hipGetLastError();
}

hipError_t launch_ring_step(const RingArgs &a, int bf16, int head_dim, hipStream_t s) {
  if (a.units == 0) return hipSuccess;
  if (bf16) return head_dim == 128 ? launch_t<true, 128>(a, s) : launch_t<true, 64>(a, s);
  return head_dim == 128 ? launch_t<false, 128>(a, s) : launch_t<false, 64>(a, s);
}

}  // namespace kvev
