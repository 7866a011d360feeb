// score.hip -- per-token eviction scores of a paged KV cache (gfx950).
//
// One workgroup (4 or 8 waves) scores a tile of consecutive 16-token
// blocks of one KV head (b, h).  The G*W observation-window query rows of the
// head's GQA group are staged once in LDS in MFMA fragment order; each wave
// streams its own key blocks straight from HBM into registers (16-byte loads,
// the four lane groups of a key row reading 64 contiguous bytes each) and
// computes
//     s = q.k       on v_mfma_f32_16x16x32_bf16 (fp32 caches: 16x16x4 f32)
//     p = exp(scale*s - lse) = exp2(s*c1 - lse*log2e), 0 when pos > q_pos
// then reduces p over the rows in a fixed order (per lane, then across the
// four lane groups).  The SnapKV max-pool needs r neighbours on each side: a
// tile also scores ceil(r/16) halo blocks on either side, so the pool is
// finished in LDS without any exchange between workgroups ([SNAP] "How it
// works").  No float atomics: results are bitwise reproducible.
//
// DropKV ([DROP] "The news", Lemma 1: removing key j moves the renormalised
// output by p_j/(1-p_j)*(a - v_j); the score is the length of that shift,
// summed over the window) also streams the value blocks.  `a` is the forward
// pass's fp32 output; for bf16 caches it is staged as a bf16 high part and a
// bf16 low part (a - hi), so a.v = hi.v + lo.v on the same MFMA tiles keeps
// 16 of a's 24 mantissa bits.  ||a||^2 comes from the fp32 values, ||v||^2
// from the diagonal of each value block's Gram matrix (MFMA), and the a.v
// accumulator starts at -(||a||^2 + ||v||^2)/2, so that it ends at
//     -X/2,  X = ||a - v||^2 = ||a||^2 - 2 a.v + ||v||^2   (clamped at 0)
// ([DROP] "Why does the Triton kernel matter?": the expansion lets each value
// tile be read once).  Where every weight of a wave's 16 x 32 tile is below
// 2^-12, term = (p + p^2) * sqrt(X) (p/(1-p) to within a relative p^2 < 2^-24;
// two transcendentals per element, exp2 and sqrt); otherwise
// term = p * X * rsq(X * (1-p)^2).
// For p >= 1/4 the term is sensitive to the rounding of x = scale*s - lse
// (its relative error grows as 1/(1-p)) and the expansion cancels as a
// approaches v_j, so those (row, key) pairs, at most four per row when the
// LSE is the row's own, are queued in LDS (in a fixed order: row tile, block,
// row, lane) and, once the streaming loop is done, recomputed exactly: q.k
// and ||a - v||^2 in double over the row, in ascending d, x in double,
// 1 - p = -expm1(x), +inf when x >= 0.  Each key's exact terms are added to
// its row sum in queue order.  The queue holds four entries per staged row;
// a workgroup with more such pairs (only an LSE below the rows' own gets
// there; the count depends on the data alone) streams its blocks again and
// keeps the expansion's value for every pair.
//
// Large windows whose rows do not fit in LDS are split over several
// workgroups per tile (the parts of a tile are adjacent on one XCD, so they
// share its L2 for the key and value blocks); each writes its rows' raw sums
// to the workspace, and a combine pass adds the parts in order and applies
// ACCUMULATE, the pool and the histogram.
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

// min(v, 0) for any v that is not a NaN (a NaN gives 0, as fmaxf(-v, 0)
// would), as one integer min on the bits: a negative float is a negative
// integer, any other is not.
__device__ __forceinline__ float min_zero(float v) {
  return __int_as_float(min(__float_as_int(v), 0));
}

// fp32 -> bf16 bits, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint32_t bf16_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// The DropKV term of one (window row, key) pair from its definition, in
// double: the q.k dot product and ||a - v||^2 over the rows in ascending d,
// x = scale*s - lse, p = exp(x), 1 - p = -expm1(x); +inf when x >= 0.
template <bool BF16, int D>
__device__ __forceinline__ float drop_term_exact(const uint8_t *qrow, const float *arow,
                                                           const uint8_t *krow,
                                                           const uint8_t *vrow, float scale,
                                                           float lse) {
  auto elem = [](const uint8_t *row, int d) -> double {
    if constexpr (BF16)
      return (double)__uint_as_float((uint32_t)reinterpret_cast<const uint16_t *>(row)[d] << 16);
    else
      return (double)reinterpret_cast<const float *>(row)[d];
  };
  double dot = 0.0, r2 = 0.0;
  for (int d = 0; d < D; ++d) {
    dot += elem(qrow, d) * elem(krow, d);
    const double diff = (double)arow[d] - elem(vrow, d);
    r2 += diff * diff;
  }
  const double x = (double)scale * dot - (double)lse;
  if (x >= 0.0) return __builtin_inff();
  return (float)(exp(x) / -expm1(x) * sqrt(r2));
}

}  // namespace

template <bool BF16, int D, bool DROP, int kThreads>
__global__ __launch_bounds__(kThreads) void score_kernel(const ScoreArgs P) {
  constexpr int kWaves = kThreads / kWave;
  using G_ = Geo<BF16, D>;
  constexpr int ROWB = G_::ROWB, U = G_::U;
  constexpr int NB = 2;  // key blocks per pipeline stage (two stages in flight)
  constexpr int AF = DROP ? (BF16 ? 2 : 1) : 0;  // staged copies of a: hi and lo, or fp32

  extern __shared__ __align__(16) uint8_t smem[];

  const int RT = P.rt_part;  // row tiles this workgroup stages
  // Per row tile, its fragments side by side (q, then a: hi and lo, or
  // fp32), and its per-row values side by side (LSE in log2 units, query
  // position, ||a||^2): one pointer each walks the row tiles.
  constexpr int NC = 1 + AF;            // staged fragment copies per row tile
  constexpr int NS = DROP ? 3 : 2;      // per-row values per row tile
  uint4 *frag = reinterpret_cast<uint4 *>(smem);
  float *rowd = reinterpret_cast<float *>(frag + (size_t)RT * NC * U * kWave);
  auto fragu = [&](int rt, int c, int j) { return frag + ((size_t)(rt * NC + c) * U + j) * kWave; };
  auto rowv = [&](int r, int k) { return rowd + ((r >> 4) * NS + k) * 16 + (r & 15); };
  float *S_lds = rowd + RT * NS * 16;
  const int span_blocks = P.tile_blocks + 2 * P.halo_blocks;
  float *D_lds = S_lds + span_blocks * 16;
  // DropKV's exact-term queue: entry = window row << 16 | span slot, its term
  const int qcap = DROP ? RT * 16 * kExactPerRow : 0;
  uint32_t *xq = reinterpret_cast<uint32_t *>(D_lds + (DROP ? span_blocks * 16 : 0));
  float *xt = reinterpret_cast<float *>(xq + qcap);
  uint32_t *xq_n = reinterpret_cast<uint32_t *>(xt + qcap);
  uint32_t *hl = reinterpret_cast<uint32_t *>(
      smem + ((score_lds_bytes(BF16, D, DROP, RT, P.tile_blocks, P.halo_blocks, 0) + 15) &
              ~size_t(15)));  // tile histogram (with P.hist)

  const int wg = remap_xcd(blockIdx.x, gridDim.x);
  const int part = wg % P.row_parts;
  const int wt = wg / P.row_parts;
  const int u = wt / P.tiles_per_head;
  const int tile = wt % P.tiles_per_head;
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
  const int rb = part * RT * 16;  // this workgroup's first window row of the group
  const size_t row0 = ((size_t)b * Hq + (size_t)h * P.G) * P.W + rb;  // its first row
  const int rows = min(P.rows - rb, RT * 16);  // rows it scores (>= 1)
  const uint8_t *qsrc = P.q + row0 * ROWB;
  const float *asrc = DROP ? P.a + row0 * D : nullptr;

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
  const int qpos_v = P.q_pos[(size_t)b * P.W + ((rb + lrow) % P.W)];
  const int qpw = P.q_pos[(size_t)b * P.W + min(l, P.W - 1)];
  const int npairs = RT * U;  // (row tile, chunk) pairs: 64 LDS units each
  auto stage_pair = [&](int pr_) {
    const int rt = pr_ / U, j = pr_ % U;
    const int r = min(rt * 16 + lr, rows - 1), cc = lg * U + j;
    ld16_to_lds(qsrc + (size_t)r * ROWB + cc * 16, fragu(rt, 0, j));
    if constexpr (DROP && !BF16)  // fp32 caches: a's fp32 rows are the fragments
      ld16_to_lds(reinterpret_cast<const uint8_t *>(asrc) + (size_t)r * ROWB + cc * 16,
                  fragu(rt, 1, j));
  };
  if (n <= 0 || n > max_slots) return;  // empty or inconsistent head: nothing to score
  const int nb = (n + kBlock - 1) / kBlock;
  if (tb0 >= nb) return;
  const bool split = P.row_parts > 1;
  const bool want_hist = !split && P.hist != nullptr && n > P.sel_budget;
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
    int id[NB];
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
      F.id[i] = id;
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
    *rowv(threadIdx.x, 0) = live ? lse_v * kLog2e : __builtin_inff();  // padding rows: p = 0
    *reinterpret_cast<int *>(rowv(threadIdx.x, 1)) = live ? qpos_v : INT_MAX;
  }
  for (int pr_ = wv + kQ * kWaves; pr_ < npairs; pr_ += kWaves) stage_pair(pr_);  // large windows
  for (int r = threadIdx.x + kThreads; r < RT * 16; r += kThreads) {
    const bool live = r < rows;
    const int rr = min(r, rows - 1);
    *rowv(r, 0) = live ? P.lse[row0 + rr] * kLog2e : __builtin_inff();
    *reinterpret_cast<int *>(rowv(r, 1)) =
        live ? P.q_pos[(size_t)b * P.W + ((rb + rr) % P.W)] : INT_MAX;
  }
  if constexpr (DROP) {
    if constexpr (BF16) {
      // a's fp32 rows as bf16 high and low parts, in fragment order: unit x
      // of pair x / 64 holds 8 elements of row rt*16 + (x%64)%16
      for (int x = threadIdx.x; x < RT * U * kWave; x += kThreads) {
        const int pr_ = x / kWave, ln = x % kWave;
        const int rt = pr_ / U, j = pr_ % U;
        const int r = min(rt * 16 + (ln & 15), rows - 1), cc = (ln >> 4) * U + j;
        const float4 f0 = *reinterpret_cast<const float4 *>(asrc + (size_t)r * D + cc * 8);
        const float4 f1 = *reinterpret_cast<const float4 *>(asrc + (size_t)r * D + cc * 8 + 4);
        const float fv[8] = {f0.x, f0.y, f0.z, f0.w, f1.x, f1.y, f1.z, f1.w};
        uint32_t hw[4], lw[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t h0 = bf16_bits(fv[2 * i]), h1 = bf16_bits(fv[2 * i + 1]);
          const uint32_t l0 = bf16_bits(fv[2 * i] - __uint_as_float(h0 << 16));
          const uint32_t l1 = bf16_bits(fv[2 * i + 1] - __uint_as_float(h1 << 16));
          hw[i] = h0 | (h1 << 16);
          lw[i] = l0 | (l1 << 16);
        }
        fragu(rt, 1, j)[ln] = make_uint4(hw[0], hw[1], hw[2], hw[3]);
        fragu(rt, 2, j)[ln] = make_uint4(lw[0], lw[1], lw[2], lw[3]);
      }
    }
    // ||a||^2 of each row from its fp32 values, d ascending
    for (int r = threadIdx.x; r < RT * 16; r += kThreads) {
      float ss = 0.f;
      if (r < rows) {
        const float4 *ar = reinterpret_cast<const float4 *>(asrc + (size_t)r * D);
#pragma unroll 4
        for (int d4 = 0; d4 < D / 4; ++d4) {
          const float4 f = ar[d4];
          ss = fmaf(f.x, f.x, ss);
          ss = fmaf(f.y, f.y, ss);
          ss = fmaf(f.z, f.z, ss);
          ss = fmaf(f.w, f.w, ss);
        }
      }
      *rowv(r, 2) = ss;
    }
  }
  if (want_hist)
    for (int i = threadIdx.x; i < kSelectBins; i += kThreads) hl[i] = 0;
  if (DROP && threadIdx.x == 0) *xq_n = 0;
  // earliest window query: keys at or before it are never masked
  int minq = qpw;
  for (int w = l + kWave; w < P.W; w += kWave) minq = min(minq, P.q_pos[(size_t)b * P.W + w]);
#pragma unroll
  for (int o = kWave / 2; o >= 1; o >>= 1) minq = min(minq, __shfl_xor(minq, o));
  __syncthreads();

  int fast_only = 0;  // set on a full exact-term queue: every pair by the expansion
  const bool want_sum = !DROP || (P.flags & 3) != 0;  // window sums are an output
  auto compute = [&](const Frag &F, int cur) {
    float psum[NB], pdrop[NB], hv[NB];
    bool need_mask = false;
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      psum[i] = 0.f;
      pdrop[i] = 0.f;
      hv[i] = 0.f;
      need_mask |= F.kp[i] > minq;
      if constexpr (DROP) {
        // ||v||^2 of the block's 16 keys: the diagonal of its value Gram
        // matrix on the MFMA; entry (j, j) sits in lane j + 16*(j/4), element j%4
        floatx4 g = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < U; ++j) g = mfma_unit<BF16>(F.v[i][j], F.v[i][j], g);
        const int ed = lr & 3;
        const float dg = ed == 0 ? g[0] : ed == 1 ? g[1] : ed == 2 ? g[2] : g[3];
        hv[i] = -0.5f * __shfl(dg, lr + 16 * (lr >> 2));  // -||v||^2 / 2 of key lr
      }
    }
    need_mask = __any(need_mask);

    for (int rt = 0; rt < RT; ++rt) {
      uint4 qa[U], aa[U], al[U];
#pragma unroll
      for (int j = 0; j < U; ++j) {
        qa[j] = fragu(rt, 0, j)[l];
        if constexpr (DROP) aa[j] = fragu(rt, 1, j)[l];
        if constexpr (DROP && BF16) al[j] = fragu(rt, 2, j)[l];
      }
      const float4 L = *reinterpret_cast<const float4 *>(rowv(rt * 16 + lg * 4, 0));
      const float Le[4] = {L.x, L.y, L.z, L.w};
      // acc = q.k; av starts at -(||a||^2 + ||v||^2)/2 and ends at -||a - v||^2/2
      floatx4 acc[NB], av[NB];
      if constexpr (DROP) {
        const float4 A2 = *reinterpret_cast<const float4 *>(rowv(rt * 16 + lg * 4, 2));
        const float Ae[4] = {A2.x, A2.y, A2.z, A2.w};
#pragma unroll
        for (int i = 0; i < NB; ++i)
#pragma unroll
          for (int e = 0; e < 4; ++e) av[i][e] = fmaf(Ae[e], -0.5f, hv[i]);
      }
#pragma unroll
      for (int i = 0; i < NB; ++i) acc[i] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < U; ++j) {
#pragma unroll
        for (int i = 0; i < NB; ++i) {
          acc[i] = mfma_unit<BF16>(qa[j], F.k[i][j], acc[i]);
          if constexpr (DROP) av[i] = mfma_unit<BF16>(aa[j], F.v[i][j], av[i]);
          if constexpr (DROP && BF16) av[i] = mfma_unit<BF16>(al[j], F.v[i][j], av[i]);
        }
      }
      // x = log2 p; keys after a row's query get x = -inf (p = 0)
      float x[NB][4];
#pragma unroll
      for (int i = 0; i < NB; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) x[i][e] = fmaf(acc[i][e], c1, -Le[e]);
      if (need_mask) {
        const int4 Qp = *reinterpret_cast<const int4 *>(rowv(rt * 16 + lg * 4, 1));
        const int Qe[4] = {Qp.x, Qp.y, Qp.z, Qp.w};
#pragma unroll
        for (int i = 0; i < NB; ++i)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (F.kp[i] > Qe[e]) x[i][e] = -__builtin_inff();
      }
      if constexpr (!DROP) {
#pragma unroll
        for (int i = 0; i < NB; ++i)
#pragma unroll
          for (int e = 0; e < 4; ++e) psum[i] += __builtin_amdgcn_exp2f(x[i][e]);
      } else {
        // a weight of at least 2^-12 in the wave (the lane's largest x)
        float hx = x[0][0];
#pragma unroll
        for (int i = 0; i < NB; ++i)
#pragma unroll
          for (int e = 0; e < 4; ++e) hx = fmaxf(hx, x[i][e]);
        // this row tile's terms and weights per key, added to the running
        // sums after either branch (the branches carry only these)
        float dd[NB], ds[NB];
#pragma unroll
        for (int i = 0; i < NB; ++i) dd[i] = ds[i] = 0.f;
        if (!__any(hx >= -12.f)) {
          // p < 2^-12: p/(1-p) = p + p^2 within a relative p^2 (< 2^-24);
          // the sums hold term/sqrt(2): sqrt(-av) = ||a - v|| / sqrt(2)
          float pp[NB][4];
#pragma unroll
          for (int i = 0; i < NB; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) pp[i][e] = __builtin_amdgcn_exp2f(x[i][e]);
          if (want_sum) {
#pragma unroll
            for (int i = 0; i < NB; ++i)
#pragma unroll
              for (int e = 0; e < 4; ++e) ds[i] += pp[i][e];
          }
#pragma unroll
          for (int i = 0; i < NB; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e)
              dd[i] = fmaf(fmaf(pp[i][e], pp[i][e], pp[i][e]),
                           __builtin_amdgcn_sqrtf(-min_zero(av[i][e])), dd[i]);
        } else {
          uint32_t slow = 0;  // terms with p >= 1/4: queued for the exact pass
#pragma unroll
          for (int i = 0; i < NB; ++i) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float p = __builtin_amdgcn_exp2f(x[i][e]);
              if (want_sum) ds[i] += p;
              // only the wave's own blocks queue (clamped re-reads are dropped)
              const bool exact = !fast_only && x[i][e] >= -2.f && cur + i < wb1;
              slow |= (exact ? 1u : 0u) << (i * 4 + e);
              const float X = -min_zero(av[i][e]);  // ||a - v||^2 / 2
              const float om = 1.f - p;
              const float t = p * X * __builtin_amdgcn_rsqf(fmaxf(X * om * om, __FLT_MIN__));
              dd[i] += exact ? 0.f : t;
            }
          }
          if (__any(slow != 0)) {
            // one reservation per (block, row) bit; lanes in ascending order
#pragma unroll
            for (int i = 0; i < NB; ++i) {
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const bool mine = (slow >> (i * 4 + e)) & 1u;
                const uint64_t m = __ballot(mine);
                if (m == 0) continue;
                int base = 0;
                if (l == 0) base = (int)atomicAdd(xq_n, (uint32_t)__popcll(m));
                base = __shfl(base, 0);
                const int idx = base + __popcll(m & ((1ull << l) - 1ull));
                if (mine && idx < qcap)  // window row (< rows: padding rows have p = 0), span slot
                  xq[idx] = ((uint32_t)(rt * 16 + lg * 4 + e) << 16) |
                            (uint32_t)((cur + i - cb0) * kBlock + lr);
              }
            }
          }
        }
#pragma unroll
        for (int i = 0; i < NB; ++i) {
          psum[i] += ds[i];
          pdrop[i] += dd[i];
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
        dv *= 1.41421356237309515f;  // back from term/sqrt(2)
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

  // two fragment sets: the next blocks stream in while the current ones are
  // scored; a second pass, without the exact terms, after a queue overflow
  for (;;) {
    if (nwb > 0) {
      if (fast_only) issue(F0, wb0);
      for (int cur = wb0; cur < wb1; cur += 2 * NB) {
        issue(F1, cur + NB);
        compute(F0, cur);
        issue(F0, cur + 2 * NB);
        if (cur + NB < wb1) compute(F1, cur + NB);
      }
    }
    __syncthreads();
    if (!DROP || fast_only || (int)*xq_n <= qcap) break;
    fast_only = 1;
  }

  // ---- DropKV's exact terms: one queue entry per thread, then each slot's
  // terms added to its row sum in queue order by the thread holding its first
  if constexpr (DROP) {
    const int nq = fast_only ? 0 : (int)*xq_n;
    if (nq > 0) {
      for (int e = threadIdx.x; e < nq; e += kThreads) {
        const uint32_t ent = xq[e];
        const int sl = (int)(ent & 0xffffu), r = (int)(ent >> 16);
        int id = bt[cb0 + sl / kBlock];
        id = (id >= 0 && id < P.num_blocks) ? id : 0;  // a bad id's slot is NaN anyway
        const size_t krow = ((size_t)id * kBlock + sl % kBlock) * ROWB;
        xt[e] = drop_term_exact<BF16, D>(qsrc + (size_t)r * ROWB, asrc + (size_t)r * D,
                                         P.k_pool + krow, P.v_pool + krow, P.scale,
                                         P.lse[row0 + r]);
      }
      __syncthreads();
      for (int e = threadIdx.x; e < nq; e += kThreads) {
        const uint32_t sl = xq[e] & 0xffffu;
        bool first = true;
        for (int f = 0; f < e && first; ++f) first = (xq[f] & 0xffffu) != sl;
        if (!first) continue;
        float v = D_lds[sl];
        for (int f = e; f < nq; ++f)
          if ((xq[f] & 0xffffu) == sl) v += xt[f];
        D_lds[sl] = v;
      }
      __syncthreads();
    }
  }

  // ---- outputs for the tile's own slots [s0, s1): thread t owns 8
  // consecutive slots (two 16-byte stores when the row is aligned)
  const int s0 = tb0 * kBlock, s1 = min(tb1 * kBlock, n);
  const int base = cb0 * kBlock, span_end = cb1 * kBlock;  // S_lds holds slots [base, span_end)
  const size_t orow = (size_t)u * max_slots;
  const int pr = P.pool_r;
  if (split) {
    // this part's raw sums; the combine pass finishes the scores
    const size_t prow = ((size_t)part * P.units + u) * max_slots;
    for (int s = s0 + (int)threadIdx.x; s < s1; s += kThreads) {
      if (P.part_sum) P.part_sum[prow + s] = S_lds[s - base];
      if constexpr (DROP) P.part_drop[prow + s] = D_lds[s - base];
    }
    return;
  }
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

// The scores of split windows: per 1024-slot chunk of a head, the parts'
// raw sums added in part order, then ACCUMULATE, the pool (over the summed
// window sums of [s - r, s + r]), the outputs and the selection histogram.
constexpr int kCombineThreads = 256;
constexpr int kCombineChunk = 1024;
__global__ __launch_bounds__(kCombineThreads) void score_combine_kernel(const ScoreArgs P) {
  __shared__ float S[kCombineChunk + 2 * 1024];  // the chunk and a halo of up to 1024 per side
  __shared__ uint32_t hl[kSelectBins];
  const int c = blockIdx.x, u = blockIdx.y, tid = threadIdx.x;
  const int n = P.seq_len[u];
  const int max_slots = P.max_blocks * kBlock;
  if (n <= 0 || n > max_slots) return;
  const int s0 = c * kCombineChunk;
  if (s0 >= n) return;
  const int s1 = min(s0 + kCombineChunk, n);
  const int r = (P.flags & 2) ? P.pool_r : 0;
  const int h0 = max(0, s0 - r), h1 = min(n, s1 + r);  // summed slots [h0, h1)
  const size_t orow = (size_t)u * max_slots;
  const size_t pstride = (size_t)P.units * max_slots;
  const bool want_hist = P.hist != nullptr && n > P.sel_budget;
  const int sel_nc = n - P.sel_recent;
  if (want_hist)
    for (int i = tid; i < kSelectBins; i += kCombineThreads) hl[i] = 0;
  if (P.part_sum) {
    for (int s = h0 + tid; s < h1; s += kCombineThreads) {
      float v = P.part_sum[orow + s];
      for (int p = 1; p < P.row_parts; ++p) v += P.part_sum[p * pstride + orow + s];
      S[s - h0] = v;
    }
  }
  __syncthreads();
  for (int s = s0 + tid; s < s1; s += kCombineThreads) {
    float sel = 0.f;
    if (P.flags & 1) {
      float v = S[s - h0];
      if (P.flags & 8) v += P.prev[orow + s];
      P.sum[orow + s] = v;
      sel = v;
    }
    if (P.flags & 2) {
      const int lo = max(0, s - r), hi = min(n - 1, s + r);
      float mx = S[lo - h0];
      for (int i = lo + 1; i <= hi; ++i) mx = fmaxf(mx, S[i - h0]);
      P.pooled[orow + s] = mx;
      sel = mx;
    }
    if (P.part_drop) {
      float v = P.part_drop[orow + s];
      for (int p = 1; p < P.row_parts; ++p) v += P.part_drop[p * pstride + orow + s];
      P.drop[orow + s] = v;
      sel = v;
    }
    if (want_hist && s < sel_nc) atomicAdd(&hl[score_key(sel) >> 21], 1u);
  }
  if (!want_hist) return;
  __syncthreads();
  uint32_t *hg = P.hist + (size_t)u * kSelectBins;
  for (int i = tid; i < kSelectBins; i += kCombineThreads)
    if (hl[i]) atomicAdd(&hg[i], hl[i]);
}

__host__ __device__ size_t score_lds_bytes(int bf16, int head_dim, int drop, int row_tiles,
                                            int tile_blocks, int halo_blocks, int hist) {
  const size_t rowb = (size_t)head_dim * (bf16 ? 2 : 4);
  const size_t frag = (size_t)row_tiles * 16 * rowb;  // bytes of one staged row set
  size_t bytes = frag * (drop ? (bf16 ? 3 : 2) : 1);   // q, then a (hi and lo for bf16)
  bytes += (size_t)row_tiles * 16 * 4 * (drop ? 3 : 2);
  bytes += (size_t)(tile_blocks + 2 * halo_blocks) * 16 * 4 * (drop ? 2 : 1);
  if (drop) bytes += (size_t)row_tiles * 16 * kExactPerRow * 8 + 4;  // exact-term queue
  if (hist) bytes = ((bytes + 15) & ~size_t(15)) + kSelectBins * 4;  // tile histogram
  return bytes;
}

template <bool BF16, int D, bool DROP, int T>
static hipError_t launch_t(const ScoreArgs &a, hipStream_t s) {
  const size_t lds = score_lds_bytes(BF16, D, DROP, a.rt_part, a.tile_blocks, a.halo_blocks,
                                     a.hist != nullptr && a.row_parts == 1);
  auto fn = score_kernel<BF16, D, DROP, T>;
  if (lds > 65536) {  // idempotent: set on every such launch, no cached state
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(fn),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  const unsigned grid = (unsigned)a.units * (unsigned)a.tiles_per_head * (unsigned)a.row_parts;
  hipLaunchKernelGGL(fn, dim3(grid), dim3(T), lds, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.row_parts == 1) return e;
  const int chunks = (a.max_blocks * kBlock + kCombineChunk - 1) / kCombineChunk;
  hipLaunchKernelGGL(score_combine_kernel, dim3(chunks, a.units), dim3(kCombineThreads), 0, s, a);
  return hipGetLastError();
}

template <bool BF16, int D, bool DROP>
static hipError_t launch_threads(const ScoreArgs &a, hipStream_t s) {
  // fp32 DropKV at head_dim 128 runs 256 threads only (its fragments need
  // more than the 256 registers a wave has at two waves per SIMD)
  if constexpr (!(DROP && !BF16 && D == 128))
    if (a.threads == 512) return launch_t<BF16, D, DROP, 512>(a, s);
  if (a.threads != 256) return hipErrorInvalidConfiguration;
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
