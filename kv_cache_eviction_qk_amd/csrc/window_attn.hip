// window_attn.hip -- log-sum-exp and attention output of the window queries
// (gfx950).  A stand-in for the FlashAttention-style forward pass that
// produces them, outside the eviction step ([DROP] Jargon, "Log-sum-exp";
// "Why does the Triton kernel matter?").
//
// Split over key chunks: a workgroup takes one KV head, a chunk of its keys
// and up to 256 of its G*W window rows (16-row tiles, one or two per wave;
// more rows take more workgroups per chunk).  Each step stages 32 keys (two
// 16-token blocks) in LDS: the key rows as they are, the value rows
// transposed (value d of 32 keys side by side).  Every wave then computes,
// on the MFMA,
//     S^T = K Q^T            (16 keys x 16 rows per tile; a lane holds one
//                             row's values for 8 of the 32 keys)
// keeps each row's running maximum m (log2 units: x = s * scale * log2 e)
// and the lane's share of l = sum 2^(x - m), and, when the output is wanted,
//     O^T += V^T P^T         (P = 2^(x - m), 16 d x 16 rows per tile)
// with P split into a bf16 high part and a bf16 low part for bf16 caches
// (p = hi + lo to a relative 2^-16, so a keeps fp32-class accuracy); fp32
// caches use the fp32 MFMA.  The lane's weights are the B operand as they
// stand: the value rows are transposed into LDS in the matching key order.
// l and O are rescaled only when a row's maximum grows.  A second launch
// merges the chunk partials of each row in chunk order:
//     lse = ln 2 * (M + log2 sum_c l_c 2^(m_c - M)),
//     a   = sum_c O_c 2^(m_c - M) / sum_c l_c 2^(m_c - M).
// No atomics: results are bitwise reproducible.
#include <hip/hip_runtime.h>
#include <math.h>

#include "kvev_device.h"
#include "kvev_kernels.h"

namespace kvev {

namespace {

constexpr int kKeys = 32;  // keys per step (two blocks)

template <bool BF16, int D, bool WANT_A>
struct WaGeo {
  static constexpr int EB = BF16 ? 2 : 4;
  static constexpr int ROWB = D * EB;          // bytes of one key or value row
  static constexpr int U = ROWB / 64;          // 16-byte units per lane per row
  static constexpr int CPR = ROWB / 16;        // 16-byte chunks per row
  static constexpr int KS = ROWB + 16;         // LDS stride of a staged key row
  static constexpr int VS = kKeys * EB + 16;   // LDS stride of a transposed value row
  static constexpr int KBYTES = kKeys * KS;
  static constexpr int VBYTES = WANT_A ? D * VS : 0;
  static constexpr int STAGE = KBYTES + VBYTES + kKeys * 4;  // keys, values, positions
};

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two fp32 values as packed bf16, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, bf16x2));
}

// Transposed position of key k (0..31) of a step for bf16 caches: the lane
// of lane group g holds, for its MFMA contraction slots 8g..8g+7, the keys
// 4g..4g+3 of the first block and 4g..4g+3 of the second.
__device__ __forceinline__ int vt_pos_bf16(int k) {
  const int blk = k >> 4, kk = k & 15;
  return 8 * (kk >> 2) + 4 * blk + (kk & 3);
}

}  // namespace

__host__ __device__ size_t window_attn_lds_bytes(int bf16, int head_dim, int want_a,
                                                 int chunk_slots) {
  const size_t eb = bf16 ? 2 : 4, rowb = (size_t)head_dim * eb;
  const size_t stage = kKeys * (rowb + 16) +
                       (want_a ? (size_t)head_dim * (kKeys * eb + 16) : 0) + kKeys * 4;
  return 2 * stage + (size_t)(chunk_slots / kBlock) * 4;
}

template <bool BF16, int D, bool WANT_A, int R, int kThreads>
__global__ __launch_bounds__(kThreads, 2) void window_attn_kernel(const WindowAttnArgs P) {
  using G_ = WaGeo<BF16, D, WANT_A>;
  constexpr int ROWB = G_::ROWB, U = G_::U, CPR = G_::CPR, KS = G_::KS, VS = G_::VS;
  constexpr int KBYTES = G_::KBYTES, VBYTES = G_::VBYTES, STAGE = G_::STAGE;
  constexpr int DT = D / 16;                                       // output d tiles
  constexpr int kWaves = kThreads / kWave;
  constexpr int kUnits = kKeys * CPR;                               // 16-byte units per step
  constexpr int kPer = (kUnits + kThreads - 1) / kThreads;          // per thread and tensor
  constexpr bool kGuard = kUnits % kThreads != 0;                   // some threads idle
  extern __shared__ __align__(16) uint8_t smem[];
  int *sbid = reinterpret_cast<int *>(smem + 2 * STAGE);  // the chunk's block ids

  const int chunk = blockIdx.x;
  const int u = blockIdx.y / P.row_parts, part = blockIdx.y % P.row_parts;
  const int b = u / P.Hkv, h = u % P.Hkv;
  const int l = lane_id(), lr = l & 15, lg = l >> 4;
  const int wv = threadIdx.x / kWave;
  const int max_slots = P.max_blocks * kBlock;
  int n = P.seq_len[u];
  if (n < 0 || n > max_slots) n = 0;  // inconsistent head: treated as empty
  const int j0 = chunk * P.chunk_slots;
  const int j1 = min(j0 + P.chunk_slots, n);
  const int nsteps = j1 > j0 ? (j1 - j0 + kKeys - 1) / kKeys : 0;
  const int Hq = P.Hkv * P.G;
  const size_t row0 = ((size_t)b * Hq + (size_t)h * P.G) * P.W;
  const int T = (P.rows + 15) / 16;
  const float c1 = P.scale * kLog2e;
  // a wave whose tiles all lie past the window only helps with the staging
  const bool active = (part * kWaves + wv) * R < T;
  // the window's earliest query position: keys at or before it are never masked
  int minq = P.q_pos[(size_t)b * P.W + min(lane_id(), P.W - 1)];
  for (int w = lane_id() + kWave; w < P.W; w += kWave) minq = min(minq, P.q_pos[(size_t)b * P.W + w]);
#pragma unroll
  for (int o_ = kWave / 2; o_ >= 1; o_ >>= 1) minq = min(minq, __shfl_xor(minq, o_));

  // this wave's row tiles: q fragments (lane: row lr of the tile, 16-byte
  // chunks lg*U + j), the rows' query positions
  uint4 qf[R][U];
  int qp[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int t = (part * kWaves + wv) * R + r;
    const int row = min(t * 16 + lr, P.rows - 1);
    const uint8_t *qs = P.q + (row0 + row) * ROWB;
#pragma unroll
    for (int j = 0; j < U; ++j) qf[r][j] = ld16(qs + (lg * U + j) * 16);
    qp[r] = P.q_pos[(size_t)b * P.W + (row % P.W)];
  }
  const int32_t *bt = P.block_table + (size_t)u * P.max_blocks;
  const int32_t *ps = P.pos + (size_t)u * max_slots;
  for (int i = threadIdx.x; i < P.chunk_slots / kBlock; i += kThreads) {
    const int blk = j0 / kBlock + i;
    int id = blk < P.max_blocks ? bt[blk] : -1;
    sbid[i] = (id >= 0 && id < P.num_blocks) ? id : -1;  // a bad id: its slots are skipped
  }
  // the q fragments and positions in registers before the loop: their first
  // uses sit inside it, where a wait for them would also wait for every
  // prefetch in flight, on every step
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // ---- staging: one step's 32 key rows, value rows and positions, loaded
  // into registers two steps ahead (two register sets) and written to LDS
  // one step ahead (two LDS stages)
  struct Regs {
    uint4 k[kPer], v[kPer];
    int p;
  };
  Regs RA, RB;
  // Branch-free, so that the compiler's wait before each LDS write counts
  // only the newer loads: a step past the last reloads the last one (never
  // written), idle threads reload a valid unit, every thread loads a position.
  // per thread and unit: the key of the step and the byte offset inside its block
  int ukey[kPer];
  uint32_t uoff[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int unit = kGuard ? min((int)threadIdx.x + i * kThreads, kUnits - 1)
                            : (int)threadIdx.x + i * kThreads;
    ukey[i] = unit / CPR;
    uoff[i] = (uint32_t)((ukey[i] % kBlock) * ROWB + (unit % CPR) * 16);
  }
  auto gload = [&](int s, Regs &R_) {
    uint4 *kreg = R_.k;
    uint4 *vreg = R_.v;
    const int sc = min(s, nsteps - 1);
    const int base = j0 + sc * kKeys;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int id = sbid[2 * sc + (ukey[i] >> 4)];
      const bool ok = base + ukey[i] < j1 && id >= 0;
      const size_t off = (size_t)(ok ? id : 0) * (kBlock * ROWB) + uoff[i];
      kreg[i] = ld16(P.k_pool + off);
      if constexpr (WANT_A) vreg[i] = ld16(P.v_pool + off);
    }
    {
      const int j = base + (int)threadIdx.x % kKeys;
      const bool ok = j < j1 && sbid[(j - j0) / kBlock] >= 0;
      const int pv = ps[min(j, max_slots - 1)];
      R_.p = ok ? pv : INT_MAX;  // INT_MAX: no row attends the slot
    }
  };
  auto swrite = [&](int buf, const Regs &R_) {
    const uint4 *kreg = R_.k;
    const uint4 *vreg = R_.v;
    uint8_t *st = smem + buf * STAGE;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int unit = threadIdx.x + i * kThreads;
      if (kGuard && unit >= kUnits) break;
      const int key = unit / CPR, c = unit % CPR;
      st16(st + key * KS + c * 16, kreg[i]);
      if constexpr (WANT_A) {
        uint8_t *vt = st + KBYTES;
        const uint32_t w[4] = {vreg[i].x, vreg[i].y, vreg[i].z, vreg[i].w};
        if constexpr (BF16) {  // 8 values d = 8c .. 8c+7
          const int pos = vt_pos_bf16(key);
#pragma unroll
          for (int e = 0; e < 8; ++e)
            *reinterpret_cast<uint16_t *>(vt + (8 * c + e) * VS + 2 * pos) =
                (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
        } else {  // 4 values d = 4c .. 4c+3, keys in natural order
#pragma unroll
          for (int e = 0; e < 4; ++e) *reinterpret_cast<uint32_t *>(vt + (4 * c + e) * VS + 4 * key) = w[e];
        }
      }
    }
    if ((int)threadIdx.x < kKeys) reinterpret_cast<int *>(st + KBYTES + VBYTES)[threadIdx.x] = R_.p;
  };

  float m[R], lsum[R];
  floatx4 o[R][DT];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    m[r] = -__builtin_inff();
    lsum[r] = 0.f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[r][dt] = floatx4{0.f, 0.f, 0.f, 0.f};
  }

  auto compute = [&](int s) {
    const uint8_t *st = smem + (s & 1) * STAGE;
    const int *Ps = reinterpret_cast<const int *>(st + KBYTES + VBYTES);
    const int4 P0 = *reinterpret_cast<const int4 *>(&Ps[4 * lg]);
    const int4 P1 = *reinterpret_cast<const int4 *>(&Ps[16 + 4 * lg]);
    const int kp[8] = {P0.x, P0.y, P0.z, P0.w, P1.x, P1.y, P1.z, P1.w};
    // S^T: lane holds row lr against keys 4lg+e (first block) and 16+4lg+e
    floatx4 acc[R][2];
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r][0] = acc[r][1] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const uint4 k0 = *reinterpret_cast<const uint4 *>(st + lr * KS + (lg * U + j) * 16);
      const uint4 k1 = *reinterpret_cast<const uint4 *>(st + (16 + lr) * KS + (lg * U + j) * 16);
#pragma unroll
      for (int r = 0; r < R; ++r) {
        acc[r][0] = mfma_unit<BF16>(k0, qf[r][j], acc[r][0]);
        acc[r][1] = mfma_unit<BF16>(k1, qf[r][j], acc[r][1]);
      }
    }
    // a step whose keys all sit at or before the window's earliest query needs
    // no causal mask (the common case)
    int kmax = kp[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) kmax = max(kmax, kp[e]);
    const bool need_mask = __any(kmax > minq);
    uint4 ph[R], pl[R];  // bf16: weights hi, lo; fp32: first block, second block
#pragma unroll
    for (int r = 0; r < R; ++r) {
      // x = acc * c1 (masked: -inf); without a mask the row maximum is taken
      // on acc and p = 2^(acc * c1 - m) is one fma and one exp2
      float x[8], mx;
      if (need_mask) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          x[e] = kp[e] <= qp[r] ? acc[r][e >> 2][e & 3] * c1 : -__builtin_inff();
        mx = x[0];
#pragma unroll
        for (int e = 1; e < 8; ++e) mx = fmaxf(mx, x[e]);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = acc[r][e >> 2][e & 3];
        float hi = x[0], lo = x[0];
        if (c1 >= 0.f) {
#pragma unroll
          for (int e = 1; e < 8; ++e) hi = fmaxf(hi, x[e]);
        } else {
#pragma unroll
          for (int e = 1; e < 8; ++e) lo = fminf(lo, x[e]);
        }
        mx = (c1 >= 0.f ? hi : lo) * c1;
      }
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mnew = fmaxf(m[r], mx);
      const float mref = mnew == -__builtin_inff() ? 0.f : mnew;  // nothing attended yet: p = 0
      if (__any(mnew > m[r])) {
        const float corr = __builtin_amdgcn_exp2f(m[r] - mref);  // 1 where m did not grow
        lsum[r] *= corr;
        if constexpr (WANT_A) {
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) o[r][dt] *= corr;
        }
      }
      m[r] = mnew;
      float p[8];
      if (need_mask) {
#pragma unroll
        for (int e = 0; e < 8; ++e) p[e] = __builtin_amdgcn_exp2f(x[e] - mref);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) p[e] = __builtin_amdgcn_exp2f(fmaf(x[e], c1, -mref));
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) lsum[r] += p[e];
      if constexpr (WANT_A) {
        if constexpr (BF16) {
          uint32_t hw[4], lw[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            hw[i] = pack_bf16(p[2 * i], p[2 * i + 1]);
            lw[i] = pack_bf16(p[2 * i] - __uint_as_float(hw[i] << 16),
                              p[2 * i + 1] - __uint_as_float(hw[i] & 0xffff0000u));
          }
          ph[r] = make_uint4(hw[0], hw[1], hw[2], hw[3]);
          pl[r] = make_uint4(lw[0], lw[1], lw[2], lw[3]);
        } else {
          ph[r] = make_uint4(__float_as_uint(p[0]), __float_as_uint(p[1]), __float_as_uint(p[2]),
                             __float_as_uint(p[3]));
          pl[r] = make_uint4(__float_as_uint(p[4]), __float_as_uint(p[5]), __float_as_uint(p[6]),
                             __float_as_uint(p[7]));
        }
      }
    }
    if constexpr (WANT_A) {
      const uint8_t *vt = st + KBYTES;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const uint8_t *vrow = vt + (dt * 16 + lr) * VS;
        if constexpr (BF16) {
          const uint4 va = *reinterpret_cast<const uint4 *>(vrow + lg * 16);
#pragma unroll
          for (int r = 0; r < R; ++r) {
            o[r][dt] = mfma_bf16(va, ph[r], o[r][dt]);
            o[r][dt] = mfma_bf16(va, pl[r], o[r][dt]);
          }
        } else {
          const uint4 va0 = *reinterpret_cast<const uint4 *>(vrow + 16 * lg);
          const uint4 va1 = *reinterpret_cast<const uint4 *>(vrow + 64 + 16 * lg);
#pragma unroll
          for (int r = 0; r < R; ++r) {
            o[r][dt] = mfma_f32x4(va0, ph[r], o[r][dt]);
            o[r][dt] = mfma_f32x4(va1, pl[r], o[r][dt]);
          }
        }
      }
    }
  };

  if (nsteps > 0) {
    gload(0, RA);
    gload(1, RB);
    swrite(0, RA);
  }
  __syncthreads();
  // step s: loads of step s + 2 into `ld`, scoring of stage s & 1, step s + 1
  // from `wr` into the other stage
  auto step = [&](int s, Regs &ld, const Regs &wr) {
    gload(s + 2, ld);
    if (active) compute(s);
    if (s + 1 < nsteps) swrite((s + 1) & 1, wr);
    __syncthreads();
  };
  for (int s = 0; s < nsteps; s += 2) {
    step(s, RA, RB);
    if (s + 1 < nsteps) step(s + 1, RB, RA);
  }

  // ---- the chunk's partials of this wave's rows: m (log2 units), l, O
#pragma unroll
  for (int r = 0; r < R; ++r) {
    float lt = lsum[r];
    lt += __shfl_xor(lt, 16);
    lt += __shfl_xor(lt, 32);
    const int t = (part * kWaves + wv) * R + r;
    const int row = t * 16 + lr;
    if (t >= T || row >= P.rows) continue;
    const size_t pi = ((size_t)u * P.rows + row) * P.chunks + chunk;
    if (lg == 0) {
      P.part_m[pi] = m[r];
      P.part_l[pi] = lt;
    }
    if constexpr (WANT_A) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)  // O^T rows d = 16dt + 4lg .. +3 of row lr
        *reinterpret_cast<floatx4 *>(P.part_acc + pi * D + dt * 16 + 4 * lg) = o[r][dt];
    }
  }
}

// One thread per window row: the LSE only.
__global__ __launch_bounds__(256) void window_attn_combine_lse_kernel(const WindowAttnArgs P) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (size_t)P.units * P.rows) return;
  const int u = (int)(i / P.rows), row = (int)(i % P.rows);
  const int b = u / P.Hkv, h = u % P.Hkv;
  const size_t pbase = i * P.chunks;
  float M = -__builtin_inff();
  for (int c = 0; c < P.chunks; ++c) M = fmaxf(M, P.part_m[pbase + c]);
  float L = 0.f;
  if (M != -__builtin_inff())
    for (int c = 0; c < P.chunks; ++c) L += P.part_l[pbase + c] * exp2f(P.part_m[pbase + c] - M);
  const size_t orow = ((size_t)b * P.Hkv * P.G + (size_t)h * P.G) * P.W + row;
  P.lse_out[orow] = L > 0.f ? (M + log2f(L)) * 0.693147180559945309f : -__builtin_inff();
}

// One workgroup of D threads per window row: the LSE and the output.
template <int D>
__global__ __launch_bounds__(D) void window_attn_combine_kernel(const WindowAttnArgs P) {
  const int u = blockIdx.x / P.rows, row = blockIdx.x % P.rows;
  const int b = u / P.Hkv, h = u % P.Hkv;
  const int d = threadIdx.x;
  const size_t pbase = ((size_t)u * P.rows + row) * P.chunks;
  float M = -__builtin_inff();
  for (int c = 0; c < P.chunks; ++c) M = fmaxf(M, P.part_m[pbase + c]);
  float L = 0.f, A = 0.f;
  if (M != -__builtin_inff()) {
    for (int c = 0; c < P.chunks; ++c) {
      const float w = exp2f(P.part_m[pbase + c] - M);
      L += P.part_l[pbase + c] * w;
      A += P.part_acc[(pbase + c) * D + d] * w;
    }
  }
  const size_t orow = ((size_t)b * P.Hkv * P.G + (size_t)h * P.G) * P.W + row;
  if (d == 0) P.lse_out[orow] = L > 0.f ? (M + log2f(L)) * 0.693147180559945309f : -__builtin_inff();
  P.a_out[orow * D + d] = L > 0.f ? A / L : 0.f;  // fp32 whatever the cache dtype
}

template <bool BF16, int D, bool WANT_A, int R, int T>
static hipError_t launch_t(const WindowAttnArgs &a, hipStream_t s) {
  const size_t lds = window_attn_lds_bytes(BF16, D, WANT_A, a.chunk_slots);
  auto fn = window_attn_kernel<BF16, D, WANT_A, R, T>;
  if (lds > 65536) {  // idempotent: set on every such launch, no cached state
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(fn),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(fn, dim3(a.chunks, a.units * a.row_parts), dim3(T), lds, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (WANT_A)
    hipLaunchKernelGGL(window_attn_combine_kernel<D>, dim3(a.units * a.rows), dim3(D), 0, s, a);
  else
    hipLaunchKernelGGL(window_attn_combine_lse_kernel,
                       dim3((unsigned)(((size_t)a.units * a.rows + 255) / 256)), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <bool BF16, int D, bool WANT_A>
static hipError_t launch_shape(const WindowAttnArgs &a, hipStream_t s) {
  if (a.threads == 256 && a.rt_wave == 1) return launch_t<BF16, D, WANT_A, 1, 256>(a, s);
  if (a.threads == 256 && a.rt_wave == 2) return launch_t<BF16, D, WANT_A, 2, 256>(a, s);
  if (a.threads == 512 && a.rt_wave == 2) return launch_t<BF16, D, WANT_A, 2, 512>(a, s);
  return hipErrorInvalidConfiguration;
}

template <bool BF16, int D>
static hipError_t launch_dt(const WindowAttnArgs &a, hipStream_t s) {
  return a.want_a ? launch_shape<BF16, D, true>(a, s) : launch_shape<BF16, D, false>(a, s);
}

hipError_t launch_window_attn(const WindowAttnArgs &a, int bf16, int head_dim, hipStream_t s) {
  if (bf16) return head_dim == 128 ? launch_dt<true, 128>(a, s) : launch_dt<true, 64>(a, s);
  return head_dim == 128 ? launch_dt<false, 128>(a, s) : launch_dt<false, 64>(a, s);
}

}  // namespace kvev
