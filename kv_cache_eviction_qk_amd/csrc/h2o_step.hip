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
// One launch per step; each KV head is split over `split` 1024-thread
// workgroups (one CU streams its share of the keys at a few tens of GB/s, so
// a head alone on one CU would be bound by that):
//   part  (every workgroup of the head, a contiguous range of its blocks):
//         block ids (checked), logits of the G query rows (padded to 16)
//         against 16 keys per MFMA, the workgroup's maximum m and sum
//         l = sum exp2(logit - m) per row, and e = exp2(logit - m) of its
//         slots (the first workgroup also the new token's), published to the
//         workspace with agent-scope stores; then one agent-scope atomic on
//         the head's arrival counter;
//   final (the workgroup that arrives last): lse of each row from the
//         workgroups' (m, l) in order, p = e * exp2(m - lse) summed over the
//         rows (fixed order) and added to each running score, the minimum of
//         the packed (score key, position) of the candidates, and every
//         write of the step: each score once, the new token's K / V row,
//         position and score at the pruned slot (or slot n), seq_len on
//         append, the arrival counter reset.
// Data handed between workgroups of the launch uses agent-scope atomic
// loads and stores only, ordered by waiting for completion before the
// counter atomic; the cache itself is written by the final workgroup alone.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <type_traits>

#include "kvev_device.h"
#include "kvev_kernels.h"

namespace kvev {

namespace {
constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / kWave;             // 16
constexpr int kPer = kH2oMaxBudget / kThreads;       // slots per thread (4)
constexpr int kMaxBlocksH = kH2oMaxBudget / kBlock;  // 256
constexpr int kMaxSplit = kH2oMaxSplit;            // workgroups per head at most
constexpr int kEBatch = 8;  // e values per thread per round of loads in the final step


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

template <bool BF16, int D>
__global__ __launch_bounds__(kThreads) void h2o_step_kernel(const H2oArgs P) {
  constexpr int EB = BF16 ? 2 : 4, ROWB = D * EB, U = ROWB / 64, CPR = ROWB / 16;
  constexpr int NBK = U >= 8 ? 1 : 8 / U;  // blocks per load batch of a wave (register budget)
  // the value rows for the attention output: thread = (key group, column
  // pair), VB keys per thread per batch, the first batch loaded with the keys
  constexpr int NCP = D / 2, NKG = kThreads / NCP;
  constexpr int VB = BF16 ? 16 : 8;
  using VRaw = typename std::conditional<BF16, uint32_t, float2>::type;
  extern __shared__ float lgt[];  // part: [G][cb*16] logits (log2 units); final: [G][np] e values
  __shared__ int s_bt[kMaxBlocksH];
  __shared__ unsigned long long s_wmin[kWaves];
  __shared__ float s_m[16], s_newlg[16], s_enew[16], s_r[16 * kMaxSplit];
  __shared__ float s_snew;
  __shared__ int s_last, s_dst, s_code, s_blk;

  const int S = P.split;
  const int u = blockIdx.x / S, w = blockIdx.x % S;
  const int tid = threadIdx.x, l = lane_id(), lr = l & 15, lg = l >> 4, wv = tid / kWave;
  const int b = u / P.Hkv, h = u % P.Hkv;
  const int G = P.G, budget = P.budget;
  int32_t *bt = P.block_table + (size_t)u * P.max_blocks;
  int32_t *ps = P.pos + (size_t)u * P.max_slots;
  float *sc = P.score + (size_t)u * P.max_slots;
  uint32_t *E = P.e + (size_t)u * G * P.np;         // [G][np]: e of every slot, then the new token
  uint32_t *ML = P.ml + (size_t)u * kMaxSplit * 32;  // [split][16 m, 16 l]

  const int n = P.seq_len[u];
  const int t = P.t_pos[b];
  if (n < 0 || n > budget) {  // inconsistent head: left unchanged, no workgroup arrives
    if (w == 0 && tid == 0) P.evicted[u] = -2;
    return;
  }
  const bool append = n < budget;
  const int nb = (n + kBlock - 1) / kBlock;  // blocks holding cached tokens
  const int cb = (nb + S - 1) / S;           // blocks per part
  const int lb0 = min(w * cb, nb), lb1 = min(lb0 + cb, nb);
  const int pnb = lb1 - lb0;                 // this part's blocks (may be 0)
  const int CS = cb * kBlock;                // LDS row stride of the logits

  // ---------------------------------------------------------------- part
  const int my_id = tid < pnb ? bt[lb0 + tid] : 0;
  const int Hq = P.Hkv * G;
  const uint8_t *qbase = P.q + ((size_t)b * Hq + (size_t)h * G + min(lr, G - 1)) * ROWB;
  uint4 qa[U];
#pragma unroll
  for (int j = 0; j < U; ++j) qa[j] = ld16(qbase + (lg * U + j) * 16);
  // what the final step needs, loaded by every part so that the one
  // arriving last has it at hand: the running scores and positions of the
  // thread's slots, the new K / V row (lanes 0..CPR-1 of wave 0 hold K
  // pieces, 32..32+CPR-1 V)
  float scv[kPer];
  int psv[kPer];
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int j = tid + k * kThreads;
    scv[k] = j < n ? sc[j] : 0.f;
    psv[k] = j < n ? ps[j] : 0;
  }
  uint4 newrow = make_uint4(0u, 0u, 0u, 0u);
  if (wv == 0 && (l & 31) < CPR)
    newrow = ld16((l < 32 ? P.k_new : P.v_new) + (size_t)u * ROWB + (size_t)(l & 31) * 16);
  if (tid == 0) s_code = 0;
  __syncthreads();
  if (tid < pnb) {
    const bool bad = my_id < 0 || my_id >= P.num_blocks;
    if (bad) s_code = -4;
    s_bt[tid] = bad ? 0 : my_id;  // a bad id reads block 0; the head is refused below
  }
  __syncthreads();
  if (s_code && tid == 0) atomicOr(P.err + u, 1u);
  const int ps0 = lb0 * kBlock, pslots = max(0, min(lb1 * kBlock, n) - ps0);
  const int cp = tid % NCP, kg = tid / NCP;
  VRaw vpre[VB];
  auto load_v = [&](int j0, VRaw (&vr)[VB]) {
#pragma unroll
    for (int q = 0; q < VB; ++q) {
      const int j = min(j0 + q * NKG, max(pslots - 1, 0));  // past the end: a repeat, not used
      const size_t row = (size_t)s_bt[j / kBlock] * kBlock + j % kBlock;
      vr[q] = *reinterpret_cast<const VRaw *>(P.v_pool + row * ROWB + cp * sizeof(VRaw));
    }
  };
  if (P.attn && pslots > 0) load_v(kg, vpre);
  // the new token's value at column tid % D (part 0 adds e_new * v_new)
  float vnew = 0.f;
  if (P.attn && w == 0) {
    const int d = tid % D;
    if constexpr (BF16)
      vnew = __uint_as_float((uint32_t)reinterpret_cast<const uint16_t *>(P.v_new + (size_t)u * ROWB)[d] << 16);
    else
      vnew = reinterpret_cast<const float *>(P.v_new + (size_t)u * ROWB)[d];
  }

  const float c1 = P.c1;
  const size_t lane_off = (size_t)lr * ROWB + (size_t)lg * (ROWB / 4);
  if (w == 0 && wv == kWaves - 1) {
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
  for (int ib = wv; ib < pnb; ib += kWaves * NBK) {  // wave-uniform
    // up to NBK blocks in flight; none past the part's last (each 16-byte
    // load of this layout touches 32 cache lines, so address processing,
    // not bandwidth, bounds a burst of them)
    uint4 kf[NBK][U];
    int kp[NBK];
#pragma unroll
    for (int i = 0; i < NBK; ++i) {
      const int lb = ib + i * kWaves;
      if (lb < pnb) {
        const uint8_t *src = P.k_pool + (size_t)s_bt[lb] * kBlock * ROWB + lane_off;
#pragma unroll
        for (int j = 0; j < U; ++j) kf[i][j] = ld16(src + 16 * j);
        kp[i] = ps[(lb0 + lb) * kBlock + lr];
      }
    }
#pragma unroll
    for (int i = 0; i < NBK; ++i) {
      const int lb = ib + i * kWaves;
      if (lb >= pnb) break;
      floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < U; ++j) acc = mfma_unit<BF16>(qa[j], kf[i][j], acc);
      const int slot = (lb0 + lb) * kBlock + lr;
      const bool live = slot < n && kp[i] <= t;  // later positions are not attended
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (4 * lg + e < G) lgt[(4 * lg + e) * CS + lb * kBlock + lr] = live ? acc[e] * c1 : -__builtin_inff();
    }
  }
  __syncthreads();
  // the part's maximum and sum per row (one wave per row), then e of its slots
  for (int g = wv; g < G; g += kWaves) {
    const float *row = lgt + (size_t)g * CS;
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
    if (w == 0 && mx != -__builtin_inff()) z += __builtin_amdgcn_exp2f(s_newlg[g] - mx);
    if (l == 0) {
      s_m[g] = mx;
      cst(ML + w * 32 + g, __float_as_uint(mx));
      cst(ML + w * 32 + 16 + g, __float_as_uint(z));
      const float enew = w == 0 ? __builtin_amdgcn_exp2f(s_newlg[g] - mx) : 0.f;
      s_enew[g] = enew;
      if (w == 0) cst(E + (size_t)g * P.np + n, __float_as_uint(enew));
    }
  }
  __syncthreads();
  for (int i = tid; i < G * pslots; i += kThreads) {
    const int g = i / pslots, j = i % pslots;
    const float m = s_m[g];
    const float e = m == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(lgt[(size_t)g * CS + j] - m);
    cst(E + (size_t)g * P.np + ps0 + j, __float_as_uint(e));
    if (P.attn) lgt[(size_t)g * CS + j] = e;  // the P.V product below reads them
  }
  if (P.attn) {
    // the part's share of the attention output, o[g][d] = sum_j e[g][j] v[j][d]
    // (plus e_new v_new in part 0), in fp32 on the VALU: thread = (key
    // group, column pair); a wave reads whole value rows; rows four at a
    // time; the key groups summed in order through LDS
    __syncthreads();
    float *red = lgt + (size_t)G * P.np;  // [NKG][4][D], after the e values
    float *O = P.o + ((size_t)u * kMaxSplit + w) * G * D;
    for (int g0 = 0; g0 < G; g0 += 4) {
      float a0[4] = {0.f, 0.f, 0.f, 0.f}, a1[4] = {0.f, 0.f, 0.f, 0.f};
      for (int j0 = kg; j0 < pslots; j0 += NKG * VB) {
        VRaw vr[VB];
        if (j0 == kg) {
#pragma unroll
          for (int q = 0; q < VB; ++q) vr[q] = vpre[q];
        } else {
          load_v(j0, vr);  // heads longer than one batch per part
        }
        // branch-free, so the LDS reads of the batch can all be in flight:
        // keys past the part and rows past G read a valid address and weigh 0
#pragma unroll
        for (int q = 0; q < VB; ++q) {
          const int j = j0 + q * NKG;
          const bool jin = j < pslots;
          const int jc = jin ? j : 0;
          float v0, v1;
          if constexpr (BF16) {
            v0 = __uint_as_float(vr[q] << 16);
            v1 = __uint_as_float(vr[q] & 0xffff0000u);
          } else {
            v0 = vr[q].x;
            v1 = vr[q].y;
          }
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const bool in = jin && g0 + r < G;
            const float e = lgt[(size_t)min(g0 + r, G - 1) * CS + jc];
            a0[r] = fmaf(in ? e : 0.f, v0, a0[r]);
            a1[r] = fmaf(in ? e : 0.f, v1, a1[r]);
          }
        }
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        red[((size_t)kg * 4 + r) * D + 2 * cp] = a0[r];
        red[((size_t)kg * 4 + r) * D + 2 * cp + 1] = a1[r];
      }
      __syncthreads();
      for (int i = tid; i < 4 * D; i += kThreads) {
        const int r = i / D, d = i % D;
        if (g0 + r >= G) continue;
        float acc = 0.f;
        for (int k = 0; k < NKG; ++k) acc += red[((size_t)k * 4 + r) * D + d];
        if (w == 0) acc = fmaf(s_enew[g0 + r], vnew, acc);  // i == tid (4 * D <= kThreads)
        cst(reinterpret_cast<uint32_t *>(O) + (size_t)(g0 + r) * D + d, __float_as_uint(acc));
      }
      __syncthreads();
    }
  }
  // every published value has completed before the arrival is counted
  drain();
  __syncthreads();
  if (tid == 0)
    s_last = __hip_atomic_fetch_add(P.arrive + u, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
             (uint32_t)(S - 1);
  __syncthreads();
  if (!s_last) return;

  // --------------------------------------------------------------- final
  // one round of loads: every part's e values (into LDS, over the logits)
  // and (m, l) of each row; thread 0 then settles the append block
  const int etot = G * P.np;
  float *EL = lgt;  // [G][np]
  auto load_e = [&](int k0) {  // kEBatch loads per thread in flight, then to LDS
    uint32_t ebuf[kEBatch];
#pragma unroll
    for (int k = 0; k < kEBatch; ++k) {
      const int i = tid + (k0 + k) * kThreads;
      ebuf[k] = i < etot ? cld(E + i) : 0u;
    }
#pragma unroll
    for (int k = 0; k < kEBatch; ++k) {
      const int i = tid + (k0 + k) * kThreads;
      if (i < etot) EL[i] = __uint_as_float(ebuf[k]);
    }
  };
  load_e(0);
  // the parts' attention shares of this thread's (row, column) outputs
  constexpr int kOPer = 16 * D / kThreads;  // outputs per thread at most (G <= 16)
  float oq[kOPer][kMaxSplit];
  if (P.attn) {
    const uint32_t *O = reinterpret_cast<const uint32_t *>(P.o + (size_t)u * kMaxSplit * G * D);
#pragma unroll
    for (int k = 0; k < kOPer; ++k) {
      const int i = tid + k * kThreads;
#pragma unroll
      for (int q = 0; q < kMaxSplit; ++q)
        oq[k][q] = (i < G * D && q < S) ? __uint_as_float(cld(O + (size_t)q * G * D + i)) : 0.f;
    }
  }
  float mq[kMaxSplit], lq[kMaxSplit];
  if (tid < G) {
#pragma unroll
    for (int q = 0; q < kMaxSplit; ++q) {
      mq[q] = q < S ? __uint_as_float(cld(ML + q * 32 + tid)) : -__builtin_inff();
      lq[q] = q < S ? __uint_as_float(cld(ML + q * 32 + 16 + tid)) : 0.f;
    }
  }
  if (tid == 0) {
    cst(P.arrive + u, 0u);  // state for the next call
    int code = 0;
    if (cld(P.err + u)) {
      cst(P.err + u, 0u);
      code = -4;
    }
    int blk = -1;
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
  for (int k0 = kEBatch; k0 * kThreads < etot; k0 += kEBatch) load_e(k0);  // large G * budget
  // lse of each row from the parts' (m, l), parts in order; r = exp2(m - lse)
  if (tid < G) {
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
      s_r[tid * kMaxSplit + q] = mq[q] == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(mq[q] - lse);
  }
  __syncthreads();
  if (s_code) {
    if (tid == 0) P.evicted[u] = s_code;
    return;
  }

  // the attention output of each query row: the parts' o combined in order
  if (P.attn) {
#pragma unroll
    for (int k = 0; k < kOPer; ++k) {
      const int i = tid + k * kThreads;
      if (i < G * D) {
        const int g = i / D;
        float acc = 0.f;
#pragma unroll
        for (int q = 0; q < kMaxSplit; ++q)
          if (q < S) acc = fmaf(oq[k][q], s_r[g * kMaxSplit + q], acc);
        P.attn[((size_t)b * Hq + (size_t)h * G) * D + i] = acc;
      }
    }
  }

  // running scores, the new token's score, the candidates' minimum
  unsigned long long best = ~0ull;
  const long long R = P.recent;
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int j = tid + k * kThreads;
    if (j < n) {
      const int q = (j / kBlock) / cb;
      float p = 0.f;
      for (int g = 0; g < G; ++g) p += EL[(size_t)g * P.np + j] * s_r[g * kMaxSplit + q];
      scv[k] += p;
      if ((long long)t - psv[k] >= R) {
        const unsigned long long c = pack_min(scv[k], psv[k]);
        best = c < best ? c : best;
      }
    }
  }
  if (tid == 0) {
    float snew = 0.f;
    for (int g = 0; g < G; ++g) snew += EL[(size_t)g * P.np + n] * s_r[g * kMaxSplit];
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
  for (int q = 1; q < kWaves; ++q) m = s_wmin[q] < m ? s_wmin[q] : m;
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

  // writes: each score once; the new token at slot dst
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
    const int blk = append ? s_blk : bt[dst / kBlock];
    const size_t row = (size_t)blk * kBlock + dst % kBlock;
    st16((l < 32 ? P.k_pool : P.v_pool) + row * ROWB + (size_t)(l & 31) * 16, newrow);
  }
}

size_t h2o_lds_bytes(const H2oArgs &a, int head_dim) {
  // the final step's e values ([G][np]) bound any part's logits ([G][cb*16]);
  // with the attention output the P.V reduction buffer ([key groups][4][D]) follows
  const size_t red = a.attn ? (size_t)kThreads / (head_dim / 2) * 4 * head_dim : 0;
  return ((size_t)a.G * a.np + red) * sizeof(float);
}

template <bool BF16, int D>
static hipError_t launch_t(const H2oArgs &a, size_t lds, hipStream_t s) {
  auto fn = h2o_step_kernel<BF16, D>;
  if (lds > 65536) {  // idempotent: set on every such launch, no cached state
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(fn),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(fn, dim3((unsigned)(a.units * a.split)), dim3(kThreads), lds, s, a);
  return hipGetLastError();
}

hipError_t launch_h2o_step(const H2oArgs &a, int bf16, int head_dim, hipStream_t s) {
  const size_t lds = h2o_lds_bytes(a, head_dim);
  if (bf16) return head_dim == 128 ? launch_t<true, 128>(a, lds, s) : launch_t<true, 64>(a, lds, s);
  return head_dim == 128 ? launch_t<false, 128>(a, lds, s) : launch_t<false, 64>(a, lds, s);
}

}  // namespace kvev
