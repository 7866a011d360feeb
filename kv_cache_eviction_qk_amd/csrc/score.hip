// score.hip -- per-token eviction scores of a paged KV cache (gfx950).
//
// One workgroup (4 or 8 waves) scores a tile of consecutive 16-token
// blocks of one KV head (b, h).  The G*W observation-window query rows of the head's GQA
// group are staged once in LDS in MFMA fragment order; each wave streams its
// own key blocks straight from HBM into registers (16-byte loads, the four
// lane groups of a key row reading 64 contiguous bytes each) and computes
//     s = q.k       on v_mfma_f32_16x16x32_bf16 (fp32 caches: 16x16x4 f32)
//     p = exp(scale*s - lse) = exp2(s*c1 - lse*log2e), 0 when pos > q_pos
// then reduces p over the rows in a fixed order (per lane, then across the
// four lane groups).  DropKV also streams the value blocks and computes
//     a.v on the same MFMA tiles, ||v||^2 on the VALU,
//     ||a - v||^2 = ||a||^2 - 2 a.v + ||v||^2  (clamped at 0)
//     term = p / (1 - p) * sqrt(||a - v||^2)     (+inf when p >= 1)
// (v_rcp_f32 and v_sqrt_f32, 1 ulp each: the correctly rounded library
// square root costs about a dozen more VALU instructions per element)
// ([DROP] "fused Triton kernels": the expansion lets each value tile be read
// once).  The SnapKV max-pool needs r neighbours on each side: a tile also
// scores ceil(r/16) halo blocks on either side, so the pool is finished in
// LDS without any exchange between workgroups ([SNAP] "How it works").
// No float atomics: results are bitwise reproducible.
//
// For the fused eviction pass the scores go to a workspace row (the output
// row is then written compacted), ACCUMULATE reads the running sums from
// their own pointer, a tile that meets a block id outside the pool flags its
// head (so that the pass leaves such a head's cache alone), and each tile
// adds the top 11 key bits of its candidate slots' scores to its head's
// histogram (LDS, then integer atomics), so the selection needs no pass of
// its own over the scores.
#include <hip/hip_runtime.h>

#include "kvev_device.h"
#include "kvev_kernels.h"

namespace kvev {

namespace {


template <bool BF16, int D>
struct Geo {
  static constexpr int EB = BF16 ? 2 : 4;   // element bytes
  static constexpr int ROWB = D * EB;       // bytes of one key / query row
  static constexpr int U = ROWB / 64;       // 16-byte units per lane per row
  static constexpr int CPR = ROWB / 16;     // 16-byte chunks per row
};

__device__ __forceinline__ int remap_xcd(int id, int n) {
  // Consecutive tiles of a head land on the same XCD (shared L2 for the
  // query rows and the halo blocks): hardware deals workgroups to the 8 XCDs
  // round robin.
  if (n % 8 != 0) return id;
  return (id % 8) * (n / 8) + id / 8;
}

}  // namespace

template <bool BF16, int D, bool DROP, int kThreads>
__global__ __launch_bounds__(kThreads) void score_kernel(const ScoreArgs P) {
  constexpr int kWaves = kThreads / kWave;
  using G_ = Geo<BF16, D>;
  constexpr int ROWB = G_::ROWB, U = G_::U, CPR = G_::CPR;
  constexpr int NB = 2;  // key blocks per pipeline stage (two stages in flight)

  extern __shared__ __align__(16) uint8_t smem[];

  const int RT = P.row_tiles;
  uint4 *qfrag = reinterpret_cast<uint4 *>(smem);
  uint4 *afrag = qfrag + RT * U * kWave;
  float *lse2 = reinterpret_cast<float *>(afrag + (DROP ? RT * U * kWave : 0));
  int *qposr = reinterpret_cast<int *>(lse2 + RT * 16);
  float *an2 = reinterpret_cast<float *>(qposr + RT * 16);
  float *S_lds = an2 + (DROP ? RT * 16 : 0);
  const int span_blocks = P.tile_blocks + 2 * P.halo_blocks;
  float *D_lds = S_lds + span_blocks * 16;
  uint32_t *hl = reinterpret_cast<uint32_t *>(
      smem + ((score_lds_bytes(BF16, D, DROP, RT, P.tile_blocks, P.halo_blocks, 0) + 15) &
              ~size_t(15)));  // tile histogram (with P.hist)

  const int wg = remap_xcd(blockIdx.x, gridDim.x);
  const int u = wg / P.tiles_per_head;
  const int tile = wg % P.tiles_per_head;
  if (u >= P.units) return;
  const int b = u / P.Hkv, h = u % P.Hkv;
  const int max_slots = P.max_blocks * kBlock;
  const int tb0 = tile * P.tile_blocks;
  // The tile's block range over the whole list (the head's length is not
  // known before the first loads return): waves split [cb0, cb1s) evenly and
  // later skip blocks past the head's last one.
  const int tb1s = min(tb0 + P.tile_blocks, P.max_blocks);
  const int cb0 = max(0, tb0 - P.halo_blocks), cb1s = min(P.max_blocks, tb1s + P.halo_blocks);
  const int l = lane_id(), lr = l & 15, lg = l >> 4;
  const int wv = threadIdx.x / kWave;
  const int nblk = cb1s - cb0;
  const int wb0 = cb0 + (nblk * wv) / kWaves, wb1s = cb0 + (nblk * (wv + 1)) / kWaves;
  const int32_t *bt = P.block_table + (size_t)u * P.max_blocks;
  const int32_t *ps = P.pos + (size_t)u * max_slots;
  const size_t lane_off = (size_t)lr * ROWB + (size_t)lg * (ROWB / 4);
  const float c1 = P.c1;
  const int Hq = P.Hkv * P.G;
  const size_t row0 = ((size_t)b * Hq + (size_t)h * P.G) * P.W;  // first row of the group
  const int rows = P.rows;
  const uint8_t *qsrc = P.q + row0 * ROWB;
  const uint8_t *asrc = DROP ? P.a + row0 * ROWB : nullptr;
  const int nunits = RT * U * kWave;  // 16-byte units of the staged rows

  // ---- one round of loads at entry, none waiting on another: the head's
  // length, this wave's block ids (one lane each; at most 64 blocks per wave),
  // the LSE and positions of the window rows.  The window rows themselves go
  // straight into LDS in MFMA fragment order (stage_pair): LDS unit
  // (rt * U + j) * 64 + lane holds row rt*16 + lane%16, 16-byte chunk
  // (lane/16) * U + j.  Indices are clamped in range; rows past the group
  // repeat the last row (their LSE is +inf, so p = 0 for them).
  const int n = P.seq_len[u];
  int my_id = bt[min(wb0 + l, P.max_blocks - 1)];
  const int lrow = min((int)threadIdx.x, rows - 1);
  const float lse_v = P.lse[row0 + lrow];
  const int qpos_v = P.q_pos[(size_t)b * P.W + (lrow % P.W)];
  const int qpw = P.q_pos[(size_t)b * P.W + min(l, P.W - 1)];
  const int npairs = RT * U;  // (row tile, chunk) pairs: 64 LDS units each
  auto stage_pair = [&](int pr_) {
    const int rt = pr_ / U, j = pr_ % U;
    const int r = min(rt * 16 + lr, rows - 1), cc = lg * U + j;
    ld16_to_lds(qsrc + (size_t)r * ROWB + cc * 16, qfrag + (size_t)pr_ * kWave);
    if constexpr (DROP) ld16_to_lds(asrc + (size_t)r * ROWB + cc * 16, afrag + (size_t)pr_ * kWave);
  };
  if (n <= 0 || n > max_slots) return;  // empty or inconsistent head: nothing to score
  const int nb = (n + kBlock - 1) / kBlock;
  if (tb0 >= nb) return;
  const bool want_hist = P.hist != nullptr && n > P.sel_budget;
  const int sel_nc = n - P.sel_recent;  // candidate slots
  const int tb1 = min(tb0 + P.tile_blocks, nb);
  const int cb1 = min(nb, tb1 + P.halo_blocks);
  const int wb1 = min(wb1s, cb1);  // this wave's live blocks: [wb0, wb1)
  const int nwb = max(0, wb1 - wb0);
  const bool my_bad = (l < nwb) && (my_id < 0 || my_id >= P.num_blocks);
  const uint64_t bad_mask = __ballot(my_bad);
  if (my_bad) my_id = 0;  // a bad id loads block 0 and yields NaN scores
  if (bad_mask && P.head_err && l == 0) atomicOr(&P.head_err[u], 1u);

  struct Frag {
    uint4 k[NB][U];
    uint4 v[NB][U];
    int kp[NB];
  };
  // Loads of blocks [cur, cur + NB), clamped to the wave's last block so every
  // issue has the same shape (the clamped re-reads hit the cache).  A wave
  // without live blocks still issues (block 0): no branch around the loads,
  // so the compiler counts the loads in flight exactly.
  auto issue = [&](Frag &F, int cur) {
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int blk = max(wb0, min(cur + i, wb1 - 1));
      int id = __builtin_amdgcn_readlane(my_id, blk - wb0);
      id = (id >= 0 && id < P.num_blocks) ? id : 0;
      const uint8_t *ksrc = P.k_pool + (size_t)id * kBlock * ROWB + lane_off;
#pragma unroll
      for (int j = 0; j < U; ++j) F.k[i][j] = ld16(ksrc + 16 * j);
      if constexpr (DROP) {
        const uint8_t *vsrc = P.v_pool + (size_t)id * kBlock * ROWB + lane_off;
#pragma unroll
        for (int j = 0; j < U; ++j) F.v[i][j] = ld16(vsrc + 16 * j);
      }
      F.kp[i] = ps[blk * kBlock + lr];
    }
  };
  Frag F0, F1;
  issue(F0, wb0);
  // the window rows into LDS right behind the first key blocks (a load into
  // LDS issued earlier would make the compiler wait for it before any other
  // load's result is used)
  constexpr int kQ = 4;  // pairs per wave issued here (later pairs repeat the last)
#pragma unroll
  for (int q = 0; q < kQ; ++q) stage_pair(min(wv + q * kWaves, npairs - 1));

  // ---- the rest of the window-row staging while the first key blocks stream in
  if ((int)threadIdx.x < RT * 16) {
    const bool live = (int)threadIdx.x < rows;
    lse2[threadIdx.x] = live ? lse_v * kLog2e : __builtin_inff();  // padding rows: p = 0
    qposr[threadIdx.x] = live ? qpos_v : INT_MAX;
  }
  for (int pr_ = wv + kQ * kWaves; pr_ < npairs; pr_ += kWaves) stage_pair(pr_);  // large windows
  for (int r = threadIdx.x + kThreads; r < RT * 16; r += kThreads) {
    const bool live = r < rows;
    const int rr = min(r, rows - 1);
    lse2[r] = live ? P.lse[row0 + rr] * kLog2e : __builtin_inff();
    qposr[r] = live ? P.q_pos[(size_t)b * P.W + (rr % P.W)] : INT_MAX;
  }
  if constexpr (DROP) {
    // ||a||^2 of each row from the staged units, chunks in order
    __syncthreads();
    for (int r = threadIdx.x; r < RT * 16; r += kThreads) {
      const int rt = r >> 4, lr16 = r & 15;
      float ss = 0.f;
      for (int g = 0; g < 4; ++g)
        for (int j = 0; j < U; ++j) ss += sumsq_unit<BF16>(afrag[(rt * U + j) * kWave + g * 16 + lr16]);
      an2[r] = r < rows ? ss : 0.f;
    }
  }
  if (want_hist)
    for (int i = threadIdx.x; i < kSelectBins; i += kThreads) hl[i] = 0;
  // earliest window query: keys at or before it are never masked
  int minq = qpw;
  for (int w = l + kWave; w < P.W; w += kWave) minq = min(minq, P.q_pos[(size_t)b * P.W + w]);
#pragma unroll
  for (int o = kWave / 2; o >= 1; o >>= 1) minq = min(minq, __shfl_xor(minq, o));
  __syncthreads();

  auto compute = [&](const Frag &F, int cur) {
    float psum[NB], pdrop[NB], vn2[NB];
    bool need_mask = false;
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      psum[i] = 0.f;
      pdrop[i] = 0.f;
      need_mask |= F.kp[i] > minq;
      if constexpr (DROP) {
        float ss = 0.f;
#pragma unroll
        for (int j = 0; j < U; ++j) ss += sumsq_unit<BF16>(F.v[i][j]);
        ss += __shfl_xor(ss, 16);
        ss += __shfl_xor(ss, 32);
        vn2[i] = ss;  // ||v||^2 of key lr, in every lane group
      }
    }
    need_mask = __any(need_mask);

    for (int rt = 0; rt < RT; ++rt) {
      uint4 qa[U], aa[U];
#pragma unroll
      for (int j = 0; j < U; ++j) {
        qa[j] = qfrag[(rt * U + j) * kWave + l];
        if constexpr (DROP) aa[j] = afrag[(rt * U + j) * kWave + l];
      }
      const float4 L = *reinterpret_cast<const float4 *>(&lse2[rt * 16 + lg * 4]);
      const int4 Qp = *reinterpret_cast<const int4 *>(&qposr[rt * 16 + lg * 4]);
      float4 A2 = make_float4(0.f, 0.f, 0.f, 0.f);
      if constexpr (DROP) A2 = *reinterpret_cast<const float4 *>(&an2[rt * 16 + lg * 4]);
      floatx4 acc[NB], av[NB];
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        acc[i] = floatx4{0.f, 0.f, 0.f, 0.f};
        av[i] = floatx4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int j = 0; j < U; ++j) {
#pragma unroll
        for (int i = 0; i < NB; ++i) {
          acc[i] = mfma_unit<BF16>(qa[j], F.k[i][j], acc[i]);
          if constexpr (DROP) av[i] = mfma_unit<BF16>(aa[j], F.v[i][j], av[i]);
        }
      }
      const float Le[4] = {L.x, L.y, L.z, L.w};
      const int Qe[4] = {Qp.x, Qp.y, Qp.z, Qp.w};
      const float Ae[4] = {A2.x, A2.y, A2.z, A2.w};
      if (!need_mask) {
#pragma unroll
        for (int i = 0; i < NB; ++i) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float x = fmaf(acc[i][e], c1, -Le[e]);
            const float p = __builtin_amdgcn_exp2f(x);
            psum[i] += p;
            if constexpr (DROP) {
              const float X = fmaxf(fmaf(-2.f, av[i][e], Ae[e] + vn2[i]), 0.f);
              const float t = (x >= 0.f) ? __builtin_inff()
                                         : p * __builtin_amdgcn_rcpf(1.f - p) * __builtin_amdgcn_sqrtf(X);
              pdrop[i] += t;
            }
          }
        }
      } else {
#pragma unroll
        for (int i = 0; i < NB; ++i) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const bool live = F.kp[i] <= Qe[e];
            const float x = fmaf(acc[i][e], c1, -Le[e]);
            const float p = live ? __builtin_amdgcn_exp2f(x) : 0.f;
            psum[i] += p;
            if constexpr (DROP) {
              const float X = fmaxf(fmaf(-2.f, av[i][e], Ae[e] + vn2[i]), 0.f);
              float t = (x >= 0.f) ? __builtin_inff()
                                   : p * __builtin_amdgcn_rcpf(1.f - p) * __builtin_amdgcn_sqrtf(X);
              pdrop[i] += live ? t : 0.f;
            }
          }
        }
      }
    }
    // fixed-order reduction over the four lane groups (rows 4*lg .. 4*lg+3)
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      float sv = psum[i];
      sv += __shfl_xor(sv, 16);
      sv += __shfl_xor(sv, 32);
      float dv = pdrop[i];
      if constexpr (DROP) {
        dv += __shfl_xor(dv, 16);
        dv += __shfl_xor(dv, 32);
      }
      const int blk = cur + i;
      if (blk < wb1 && lg == 0) {
        // a block id outside the pool gives NaN scores for its slots
        const bool bad = (bad_mask >> (blk - wb0)) & 1ull;
        S_lds[(blk - cb0) * kBlock + lr] = bad ? __builtin_nanf("") : sv;
        if constexpr (DROP) D_lds[(blk - cb0) * kBlock + lr] = bad ? __builtin_nanf("") : dv;
      }
    }
  };

  // two fragment sets: the next blocks stream in while the current ones are scored
  if (nwb > 0) {
    for (int cur = wb0; cur < wb1; cur += 2 * NB) {
      issue(F1, cur + NB);
      compute(F0, cur);
      issue(F0, cur + 2 * NB);
      if (cur + NB < wb1) compute(F1, cur + NB);
    }
  }
  __syncthreads();

  // ---- outputs for the tile's own slots [s0, s1): thread t owns 8
  // consecutive slots (two 16-byte stores when the row is aligned)
  const int s0 = tb0 * kBlock, s1 = min(tb1 * kBlock, n);
  const int base = cb0 * kBlock, span_end = cb1 * kBlock;  // S_lds holds slots [base, span_end)
  const size_t orow = (size_t)u * max_slots;
  const int pr = P.pool_r;
  for (int g0 = s0 + (int)threadIdx.x * 8; g0 < s1; g0 += kThreads * 8) {
    const bool full = g0 + 8 <= s1;
    float S8[8], selv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) S8[e] = S_lds[min(g0 + e, span_end - 1) - base];
    auto put8 = [&](float *dst, const float (&v)[8]) {
      float *o = dst + orow + g0;
      if (full && (reinterpret_cast<uintptr_t>(o) & 15) == 0) {
        *reinterpret_cast<float4 *>(o) = make_float4(v[0], v[1], v[2], v[3]);
        *reinterpret_cast<float4 *>(o + 4) = make_float4(v[4], v[5], v[6], v[7]);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (g0 + e < s1) o[e] = v[e];
      }
    };
    if (P.flags & 1) {  // SUM (with ACCUMULATE: add to the stored score)
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        v[e] = S8[e];
        if (P.flags & 8) v[e] += g0 + e < s1 ? P.prev[orow + g0 + e] : 0.f;
        selv[e] = v[e];
      }
      put8(P.sum, v);
    }
    if (P.flags & 2) {  // POOL: max over [s - r, s + r] clamped to [0, n - 1]
      float v[8];
      if (pr <= 8) {
        // the 8 + 2r window values from registers; slots outside [0, n) are -inf
        float w[24];
#pragma unroll
        for (int i = 0; i < 24; ++i) {
          const int sl = g0 - pr + i;
          w[i] = (i < 8 + 2 * pr && sl >= 0 && sl < n) ? S_lds[min(max(sl, base), span_end - 1) - base]
                                                        : -__builtin_inff();
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          float mx = w[e];
#pragma unroll
          for (int i = 1; i <= 16; ++i)
            if (i <= 2 * pr) mx = fmaxf(mx, w[e + i]);
          v[e] = mx;
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int sl = min(g0 + e, s1 - 1);
          const int lo = max(0, sl - pr), hi = min(n - 1, sl + pr);
          float mx = S_lds[lo - base];
          for (int i = lo + 1; i <= hi; ++i) mx = fmaxf(mx, S_lds[i - base]);
          v[e] = mx;
        }
      }
      put8(P.pooled, v);
#pragma unroll
      for (int e = 0; e < 8; ++e) selv[e] = v[e];
    }
    if constexpr (DROP) {
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = D_lds[min(g0 + e, span_end - 1) - base];
      put8(P.drop, v);
#pragma unroll
      for (int e = 0; e < 8; ++e) selv[e] = v[e];
    }
    if (want_hist) {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (g0 + e < s1 && g0 + e < sel_nc) atomicAdd(&hl[score_key(selv[e]) >> 21], 1u);
    }
  }
  if (!want_hist) return;
  __syncthreads();
  uint32_t *hg = P.hist + (size_t)u * kSelectBins;
  for (int i = threadIdx.x; i < kSelectBins; i += kThreads)
    if (hl[i]) atomicAdd(&hg[i], hl[i]);
}

__host__ __device__ size_t score_lds_bytes(int bf16, int head_dim, int drop, int row_tiles,
                                            int tile_blocks, int halo_blocks, int hist) {
  const size_t rowb = (size_t)head_dim * (bf16 ? 2 : 4);
  const size_t frag = (size_t)row_tiles * 16 * rowb;  // bytes of one staged row set
  size_t bytes = frag * (drop ? 2 : 1);
  bytes += (size_t)row_tiles * 16 * 4 * (drop ? 3 : 2);
  bytes += (size_t)(tile_blocks + 2 * halo_blocks) * 16 * 4 * (drop ? 2 : 1);
  if (hist) bytes = ((bytes + 15) & ~size_t(15)) + kSelectBins * 4;  // tile histogram
  return bytes;
}

template <bool BF16, int D, bool DROP, int T>
static hipError_t launch_t(const ScoreArgs &a, hipStream_t s) {
  const size_t lds = score_lds_bytes(BF16, D, DROP, a.row_tiles, a.tile_blocks, a.halo_blocks,
                                     a.hist != nullptr);
  auto fn = score_kernel<BF16, D, DROP, T>;
  static size_t lds_set = 0;  // largest dynamic LDS size enabled for this variant
  if (lds > 65536 && lds > lds_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(fn),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    lds_set = lds;
  }
  const unsigned grid = (unsigned)a.units * (unsigned)a.tiles_per_head;
  hipLaunchKernelGGL(fn, dim3(grid), dim3(T), lds, s, a);
  return hipGetLastError();
}

template <bool BF16, int D, bool DROP>
static hipError_t launch_threads(const ScoreArgs &a, hipStream_t s) {
  if (a.threads == 512) return launch_t<BF16, D, DROP, 512>(a, s);
  return launch_t<BF16, D, DROP, 256>(a, s);
}

hipError_t launch_score(const ScoreArgs &a, int bf16, int head_dim, int drop, hipStream_t s) {
  if (bf16) {
    if (head_dim == 128)
      return drop ? launch_threads<true, 128, true>(a, s) : launch_threads<true, 128, false>(a, s);
    return drop ? launch_threads<true, 64, true>(a, s) : launch_threads<true, 64, false>(a, s);
  }
  if (head_dim == 128)
    return drop ? launch_threads<false, 128, true>(a, s) : launch_threads<false, 128, false>(a, s);
  return drop ? launch_threads<false, 64, true>(a, s) : launch_threads<false, 64, false>(a, s);
}

}  // namespace kvev
