// policy.hip -- eviction policy variants built on the selection kernels
// (gfx950).
//
// Shared scores across heads ([H2O] "Formulating Cumulative Attention
// Scores": a token's score sums the attention it receives from every head of
// the layer, so one victim set serves all heads of a sequence).  Each head's
// score row is already summed over its GQA group; the shared row of a
// sequence adds the rows of its KV heads in fp32, heads in ascending order,
// and the ordinary selection (budget, protected recent window, equal scores
// evicting the lower position, ascending victims) runs once per sequence on
// it.  Every head of the sequence then receives the same victims.  The heads
// of a sequence must hold the same tokens in the same slots (equal lengths,
// equal positions slot by slot); a sequence that does not gets n_victims -1
// on every head.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "kvev_device.h"
#include "kvev_kernels.h"

namespace kvev {

namespace {
constexpr int kRowThreads = 256;
}  // namespace

__global__ void shared_zero_kernel(uint32_t *p, size_t n) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0;
}

// The shared row of a sequence, and its length: the common length of its
// heads, or past the capacity (refused by the selection) when the heads'
// lengths or positions differ.
__global__ __launch_bounds__(kRowThreads) void shared_row_kernel(const SharedArgs P) {
  const int b = blockIdx.y, s = blockIdx.x * kRowThreads + threadIdx.x;
  const size_t u0 = (size_t)b * P.Hkv;
  const int n0 = P.seq_len[u0];
  bool bad = n0 < 0 || n0 > P.max_slots;
  for (int h = 1; h < P.Hkv; ++h) bad |= P.seq_len[u0 + h] != n0;
  if (!bad && s < n0) {
    const int p0 = P.pos[u0 * P.max_slots + s];
    float sum = P.score[u0 * P.max_slots + s];
    for (int h = 1; h < P.Hkv; ++h) {
      sum += P.score[(u0 + h) * P.max_slots + s];
      bad |= P.pos[(u0 + h) * P.max_slots + s] != p0;
    }
    P.row[(size_t)b * P.max_slots + s] = sum;
  }
  // the length: 0 before the call (zeroed); any misaligned slot or length
  // raises it past the capacity (one atomic per wave)
  const uint64_t any_bad = __ballot(bad);
  if (lane_id() == 0 && any_bad) atomicMax(P.vseq + b, P.max_slots + 1);
  if (blockIdx.x == 0 && threadIdx.x == 0 && n0 >= 0) atomicMax(P.vseq + b, n0);
}

__global__ __launch_bounds__(256) void shared_broadcast_kernel(const SharedArgs P) {
  const int u = blockIdx.y, b = u / P.Hkv;
  const int m = P.vnv[b];
  const int i0 = blockIdx.x * 256 + threadIdx.x;
  if (i0 == 0) P.n_victims[u] = m;
  for (int i = i0; i < m; i += (int)gridDim.x * 256)
    P.victims[(size_t)u * P.max_slots + i] = P.vvict[(size_t)b * P.max_slots + i];
}

hipError_t launch_select_shared(const SharedArgs &a, hipStream_t s) {
  hipLaunchKernelGGL(shared_zero_kernel, dim3((unsigned)std::min<size_t>((a.zero_words + 255) / 256, 2048)),
                     dim3(256), 0, s, a.zero, a.zero_words);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(shared_row_kernel,
                     dim3((unsigned)((a.max_slots + kRowThreads - 1) / kRowThreads), (unsigned)a.B),
                     dim3(kRowThreads), 0, s, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((e = launch_select(a.sel, s)) != hipSuccess) return e;
  hipLaunchKernelGGL(shared_broadcast_kernel,
                     dim3((unsigned)std::min((a.max_slots + 255) / 256, 64), (unsigned)(a.B * a.Hkv)),
                     dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace kvev
