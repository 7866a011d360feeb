// window_attn.hip -- log-sum-exp and attention output of the window queries
// (gfx950).  A stand-in for the forward pass that produces them, outside
// the eviction step ([DROP] Jargon, "Log-sum-exp").
//
// Split over key chunks: each workgroup takes one KV head, 128 window rows
// (two threads per row, each owning half of head_dim) and a chunk of keys.
// Key and value blocks are staged in LDS as fp32 32 keys at a time; each
// row keeps a running maximum m, the rescaled sum l and the rescaled output
// accumulator (fp32).  A second launch merges the chunk partials per row in
// chunk order: lse = M + log(sum_c l_c exp(m_c - M)), a = sum_c acc_c
// exp(m_c - M) / that sum.
#include <hip/hip_runtime.h>
#include <math.h>

#include "kvev_device.h"
#include "kvev_kernels.h"

namespace kvev {

namespace {
constexpr int kThreads = 256;
constexpr int kRowsPerWg = kThreads / 2;
constexpr int kSub = 32;  // keys staged per step

template <bool BF16>
__device__ __forceinline__ float load_elem(const uint8_t *base, size_t idx) {
  if constexpr (BF16) {
    const uint16_t b = reinterpret_cast<const uint16_t *>(base)[idx];
    return __uint_as_float((uint32_t)b << 16);
  } else {
    return reinterpret_cast<const float *>(base)[idx];
  }
}

}  // namespace

template <bool BF16, int D>
__global__ __launch_bounds__(kThreads) void window_attn_partial_kernel(const WindowAttnArgs P) {
  constexpr int H = D / 2;
  __shared__ float Ks[kSub][D + 1];
  __shared__ float Vs[kSub][D + 1];
  __shared__ int Ps[kSub];

  const int chunk = blockIdx.x;
  const int row_groups = (P.rows + kRowsPerWg - 1) / kRowsPerWg;
  const int u = blockIdx.y / row_groups, rg = blockIdx.y % row_groups;
  const int b = u / P.Hkv, h = u % P.Hkv;
  const int tid = threadIdx.x, half = tid & 1;
  const int row = rg * kRowsPerWg + tid / 2;
  const bool row_ok = row < P.rows;
  const int Hq = P.Hkv * P.G;
  const size_t row0 = ((size_t)b * Hq + (size_t)h * P.G) * P.W;
  const int max_slots = P.max_blocks * kBlock;
  int n = P.seq_len[u];
  if (n < 0 || n > max_slots) n = 0;  // inconsistent head: treated as empty
  const int j0 = chunk * P.chunk_slots, j1 = min(j0 + P.chunk_slots, n);
  const int qp = row_ok ? P.q_pos[(size_t)b * P.W + (row % P.W)] : INT_MIN;

  float q[H], acc[H];
#pragma unroll
  for (int d = 0; d < H; ++d) {
    q[d] = row_ok ? load_elem<BF16>(P.q, (row0 + row) * D + half * H + d) : 0.f;
    acc[d] = 0.f;
  }
  float m = -__builtin_inff(), l = 0.f;
  const int32_t *bt = P.block_table + (size_t)u * P.max_blocks;
  const int32_t *ps = P.pos + (size_t)u * max_slots;

  for (int base = j0; base < j1; base += kSub) {
    __syncthreads();
    for (int i = tid; i < kSub * D; i += kThreads) {
      const int jj = i / D, d = i % D;
      const int j = base + jj;
      float kv = 0.f, vv = 0.f;
      if (j < j1) {
        const int blk = bt[j / kBlock];
        if (blk >= 0 && blk < P.num_blocks) {
          const size_t r = ((size_t)blk * kBlock + j % kBlock) * D + d;
          kv = load_elem<BF16>(P.k_pool, r);
          if (P.want_a) vv = load_elem<BF16>(P.v_pool, r);
        }
      }
      Ks[jj][d] = kv;
      Vs[jj][d] = vv;
    }
    for (int i = tid; i < kSub; i += kThreads) {
      const int j = base + i;
      Ps[i] = (j < j1) ? ps[j] : INT_MAX;
    }
    __syncthreads();
    float s[kSub];
    float mt = -__builtin_inff();
#pragma unroll
    for (int jj = 0; jj < kSub; ++jj) {
      float part = 0.f;
#pragma unroll
      for (int d = 0; d < H; ++d) part = fmaf(q[d], Ks[jj][half * H + d], part);
      part += __shfl_xor(part, 1);
      const bool live = (base + jj < j1) && (Ps[jj] <= qp);
      const float sv = live ? part * P.scale : -__builtin_inff();
      s[jj] = sv;
      mt = fmaxf(mt, sv);
    }
    const float mn = fmaxf(m, mt);
    if (mn == -__builtin_inff()) continue;  // nothing attended yet
    const float corr = expf(m - mn);        // m = -inf gives 0
    l *= corr;
    if (P.want_a) {
#pragma unroll
      for (int d = 0; d < H; ++d) acc[d] *= corr;
    }
#pragma unroll
    for (int jj = 0; jj < kSub; ++jj) {
      const float p = expf(s[jj] - mn);
      l += p;
      if (P.want_a) {
#pragma unroll
        for (int d = 0; d < H; ++d) acc[d] = fmaf(p, Vs[jj][half * H + d], acc[d]);
      }
    }
    m = mn;
  }
  if (!row_ok) return;
  const int rows_pad = row_groups * kRowsPerWg;
  const size_t pi = ((size_t)u * rows_pad + row) * P.chunks + chunk;
  if (half == 0) {
    P.part_m[pi] = m;
    P.part_l[pi] = l;
  }
  if (P.want_a) {
#pragma unroll
    for (int d = 0; d < H; ++d) P.part_acc[pi * D + half * H + d] = acc[d];
  }
}

template <bool BF16, int D>
__global__ __launch_bounds__(D) void window_attn_combine_kernel(const WindowAttnArgs P) {
  const int row_groups = (P.rows + kRowsPerWg - 1) / kRowsPerWg;
  const int rows_pad = row_groups * kRowsPerWg;
  const int u = blockIdx.x / P.rows, row = blockIdx.x % P.rows;
  const int b = u / P.Hkv, h = u % P.Hkv;
  const int d = threadIdx.x;
  const size_t pbase = ((size_t)u * rows_pad + row) * P.chunks;
  float M = -__builtin_inff();
  for (int c = 0; c < P.chunks; ++c) M = fmaxf(M, P.part_m[pbase + c]);
  float L = 0.f, A = 0.f;
  if (M != -__builtin_inff()) {
    for (int c = 0; c < P.chunks; ++c) {
      const float w = expf(P.part_m[pbase + c] - M);
      L += P.part_l[pbase + c] * w;
      if (P.want_a) A += P.part_acc[(pbase + c) * D + d] * w;
    }
  }
  const int Hq = P.Hkv * P.G;
  const size_t orow = ((size_t)b * Hq + (size_t)h * P.G) * P.W + row;
  if (d == 0) P.lse_out[orow] = (L > 0.f) ? M + logf(L) : -__builtin_inff();
  if (P.want_a) {
    P.a_out[orow * D + d] = (L > 0.f) ? A / L : 0.f;  // fp32 whatever the cache dtype
  }
}

template <bool BF16, int D>
static hipError_t launch_t(const WindowAttnArgs &a, hipStream_t s) {
  const int row_groups = (a.rows + kRowsPerWg - 1) / kRowsPerWg;
  hipLaunchKernelGGL((window_attn_partial_kernel<BF16, D>), dim3(a.chunks, a.units * row_groups),
                     dim3(kThreads), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((window_attn_combine_kernel<BF16, D>), dim3(a.units * a.rows), dim3(D), 0, s,
                     a);
  return hipGetLastError();
}

hipError_t launch_window_attn(const WindowAttnArgs &a, int bf16, int head_dim, hipStream_t s) {
  if (bf16) return head_dim == 128 ? launch_t<true, 128>(a, s) : launch_t<true, 64>(a, s);
  return head_dim == 128 ? launch_t<false, 128>(a, s) : launch_t<false, 64>(a, s);
}

}  // namespace kvev
