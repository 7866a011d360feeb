// measure.hip -- block-level waste of an eviction ([VTOK] section 2, Eq. 1
// and Fig. 1): live tokens, blocks before and after compaction, and the
// blocks at half use or less, summed over the KV heads (gfx950).
//
// One thread per logical block of a head.  Before compaction ("naive"
// eviction) block b holds min(16, n - 16b) slots minus its victims; the
// victims in [16b, 16b + 16) are counted by two binary searches in the
// head's ascending victim list.  After compaction the n' kept tokens fill
// ceil(n'/16) blocks from the front, so only the last one can be half used
// or less.  Integer sums (one atomic per wave and counter): exact.
#include <hip/hip_runtime.h>

#include "kvev_device.h"
#include "kvev_kernels.h"

namespace kvev {

namespace {
constexpr int kMeasureThreads = 256;

__device__ __forceinline__ int lower_bound(const int32_t *a, int m, int key) {
  int lo = 0, hi = m;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (a[mid] < key) lo = mid + 1; else hi = mid;
  }
  return lo;
}

__device__ __forceinline__ unsigned long long wave_sum64(unsigned long long v) {
#pragma unroll
  for (int o = kWave / 2; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
}  // namespace

__global__ void measure_zero_kernel(int64_t *out) {
  if (threadIdx.x < 6) out[threadIdx.x] = 0;
}

// grid (ceil(max_blocks / 256), units)
__global__ __launch_bounds__(kMeasureThreads) void measure_kernel(const MeasureArgs P) {
  const int u = blockIdx.y;
  const int lb = blockIdx.x * kMeasureThreads + threadIdx.x;
  const int n = P.seq_len_before[u];
  const int m = P.n_victims[u];
  const bool ok = n >= 0 && n <= P.max_slots && m >= 0 && m <= n;
  unsigned long long c[6] = {0, 0, 0, 0, 0, 0};
  if (ok) {
    const int n2 = n - m;
    const int nb = (n + kBlock - 1) / kBlock, nb2 = (n2 + kBlock - 1) / kBlock;
    if (lb < nb) {
      const int32_t *vic = P.victims + (size_t)u * P.max_slots;
      const int s0 = lb * kBlock;
      const int fill = min(kBlock, n - s0);
      const int gone = lower_bound(vic, m, s0 + kBlock) - lower_bound(vic, m, s0);
      const int live = fill - gone;
      c[1] = 1;
      c[3] = 2 * live <= kBlock ? 1 : 0;
    }
    if (lb < nb2) {
      const int live2 = min(kBlock, n2 - lb * kBlock);
      c[2] = 1;
      c[4] = 2 * live2 <= kBlock ? 1 : 0;
    }
    if (lb == 0) {
      c[0] = (unsigned long long)n2;
      c[5] = (unsigned long long)(nb - nb2);
    }
  }
  unsigned long long *out = reinterpret_cast<unsigned long long *>(P.out);
#pragma unroll
  for (int i = 0; i < 6; ++i) {
    const unsigned long long t = wave_sum64(c[i]);
    if (lane_id() == 0 && t) atomicAdd(&out[i], t);
  }
}

hipError_t launch_measure(const MeasureArgs &a, hipStream_t s) {
  hipLaunchKernelGGL(measure_zero_kernel, dim3(1), dim3(64), 0, s, a.out);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.units == 0) return e;
  const int max_blocks = a.max_slots / kBlock;
  const dim3 grid((max_blocks + kMeasureThreads - 1) / kMeasureThreads, a.units);
  hipLaunchKernelGGL(measure_kernel, grid, dim3(kMeasureThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace kvev
