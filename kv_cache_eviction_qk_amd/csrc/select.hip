// select.hip -- victims of each KV head under a budget (gfx950).
//
// Scores become order-preserving 32-bit keys (kvev::score_key).  With
// m = max(0, n - budget) victims among the candidate slots [0, nc),
// nc = n - recent, the victims are the m smallest (key, slot) pairs: equal
// scores evict the lower position first ([SNAP] "Tie-breaking").  Four
// launches:
//   hist     4096 slots of one head per workgroup: LDS histogram of the top
//            11 key bits, added into the head's 2048-bin histogram (integer
//            atomics: exact).
//   collect  4096 slots per workgroup, refine one workgroup per head: the
//            exact threshold (kvev_select_head.h).
//   emit     1024 slots per workgroup: marks the victims against the threshold,
//         prefix-sums them and writes their slots from the chunk's offset,
//         so the list is in ascending slot order.
// Integer throughout: the result depends only on the score bits.
#include <hip/hip_runtime.h>

#include "kvev_device.h"
#include "kvev_kernels.h"
#include "kvev_select_head.h"

namespace kvev {

namespace {
constexpr int kHistThreads = 1024;
constexpr int kEmitThreads = 256;
constexpr int kEmitPer = kSelectChunk / kEmitThreads;
}  // namespace

__global__ __launch_bounds__(kHistThreads) void select_hist_kernel(const SelectArgs P) {
  __shared__ uint32_t hl[kSelectBins];
  const int c = blockIdx.x, u = blockIdx.y, tid = threadIdx.x;
  const int n = P.seq_len[u];
  int budget, recent;
  if (!unit_budget(P.sel, u, budget, recent)) return;   // the head step flags it
  if (n < 0 || n > P.max_slots) return;  // inconsistent head: the head step flags it
  const int m = max(0, n - budget);
  const int nc = max(0, n - recent);  // > m whenever m > 0
  if (m == 0) return;
  const int s0 = c * kHistChunk;
  if (s0 >= nc) return;
  const int s1 = min(s0 + kHistChunk, nc);
  for (int i = tid; i < kSelectBins; i += kHistThreads) hl[i] = 0;
  __syncthreads();
  const float *row = P.score + (size_t)u * P.max_slots;
  float v[kHistChunk / kHistThreads];
#pragma unroll
  for (int q = 0; q < kHistChunk / kHistThreads; ++q) {
    const int s = s0 + q * kHistThreads + tid;
    v[q] = s < s1 ? row[s] : 0.f;
  }
#pragma unroll
  for (int q = 0; q < kHistChunk / kHistThreads; ++q) {
    const int s = s0 + q * kHistThreads + tid;
    if (s < s1) atomicAdd(&hl[score_key(v[q]) >> 21], 1u);
  }
  __syncthreads();
  uint32_t *hg = P.sel.hist + (size_t)u * kSelectBins;
  for (int i = tid; i < kSelectBins; i += kHistThreads)
    if (hl[i]) atomicAdd(&hg[i], hl[i]);
}

__global__ __launch_bounds__(kSelThreads) void select_collect_kernel(const SelectArgs P) {
  __shared__ CollectLds L;
  const int c = blockIdx.x, u = blockIdx.y;
  const int n = P.seq_len[u];
  int budget, recent;
  if (!unit_budget(P.sel, u, budget, recent)) return;
  if (n < 0 || n > P.max_slots) return;
  const int m = max(0, n - budget);
  const int nc = max(0, n - recent);
  if (m == 0 || c * kHistChunk >= nc) return;
  collect_chunk(P.sel, P.score + (size_t)u * P.max_slots, P.sel.hist + (size_t)u * kSelectBins, u,
                c, m, nc, P.max_slots, L);
}

// One workgroup per head: the exact threshold from the collected bucket.
__global__ __launch_bounds__(kSelThreads) void select_refine_kernel(const SelectArgs P) {
  extern __shared__ __align__(16) uint8_t smem[];
  RefineLds &L = *reinterpret_cast<RefineLds *>(smem);
  const int u = blockIdx.x, tid = threadIdx.x;
  const int n = P.seq_len[u];
  int budget, recent;
  const bool ok = unit_budget(P.sel, u, budget, recent);
  if (!ok || n < 0 || n > P.max_slots) {  // inconsistent head
    if (tid == 0) P.sel.n_victims[u] = -1;
    return;
  }
  const int m = max(0, n - budget);
  const int nc = max(0, n - recent);
  if (m == 0) {
    if (tid == 0) P.sel.n_victims[u] = 0;
    return;
  }
  refine_head(P.sel, P.sel.hist + (size_t)u * kSelectBins, u, m, nc, L);
}

__global__ __launch_bounds__(kEmitThreads) void select_emit_kernel(const SelectArgs P) {
  __shared__ int wave_tot[kEmitThreads / kWave];
  const int c = blockIdx.x, u = blockIdx.y, tid = threadIdx.x;
  const int n = P.seq_len[u];
  int budget, recent;
  if (!unit_budget(P.sel, u, budget, recent)) return;
  if (n < 0 || n > P.max_slots) return;
  const int m = max(0, n - budget);
  const int nc = max(0, n - recent);
  if (m == 0) return;
  const int s0 = c * kSelectChunk;
  if (s0 >= nc) return;
  const int s1 = min(s0 + kSelectChunk, nc);
  const uint32_t T = P.sel.head_sel[u * 4 + 0];
  const int cut = (int)P.sel.head_sel[u * 4 + 1];
  const uint32_t off = P.sel.chunk_off[(size_t)u * P.sel.chunks + c];
  const float *row = P.score + (size_t)u * P.max_slots;
  float sv[kEmitPer];
#pragma unroll
  for (int q = 0; q < kEmitPer; ++q) {
    const int s = s0 + tid * kEmitPer + q;
    sv[q] = s < s1 ? row[s] : 0.f;
  }
  bool vic[kEmitPer];
  int cnt = 0;
#pragma unroll
  for (int q = 0; q < kEmitPer; ++q) {
    const int s = s0 + tid * kEmitPer + q;
    const uint32_t k = score_key(sv[q]);
    vic[q] = s < s1 && (k < T || (k == T && s <= cut));
    cnt += vic[q] ? 1 : 0;
  }
  const int lane = lane_id(), wv = tid / kWave;
  const int incl = (int)wave_incl_scan((uint32_t)cnt);
  if (lane == kWave - 1) wave_tot[wv] = incl;
  __syncthreads();
  int before = 0;
  for (int w = 0; w < wv; ++w) before += wave_tot[w];
  uint32_t o = off + (uint32_t)(before + incl - cnt);
  int32_t *out = P.victims + (size_t)u * P.max_slots;
#pragma unroll
  for (int q = 0; q < kEmitPer; ++q)
    if (vic[q]) {
      if (o < (uint32_t)m) out[o] = s0 + tid * kEmitPer + q;
      ++o;
    }
}

hipError_t launch_select(const SelectArgs &a, hipStream_t s) {
  hipLaunchKernelGGL(select_hist_kernel, dim3(a.sel.nwg, a.units), dim3(kHistThreads), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(select_collect_kernel, dim3(a.sel.nwg, a.units), dim3(kSelThreads), 0, s, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(select_refine_kernel, dim3(a.units), dim3(kSelThreads), sizeof(RefineLds), s,
                     a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(select_emit_kernel, dim3(a.sel.chunks, a.units), dim3(kEmitThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace kvev
