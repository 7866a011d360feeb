// select.hip -- victims of each KV head under a budget (gfx950).
//
// One 1024-thread workgroup per KV head.  Scores become order-preserving
// 32-bit keys (kvev::score_key); an MSB-first radix select over four 8-bit
// digits finds the key T of the m-th smallest candidate and how many
// candidates equal to T are evicted (e).  Emission: each wave owns a
// contiguous run of candidate slots; a first sweep counts keys < T and
// keys == T per wave, a scan over the 16 waves gives each wave its output
// offset and its tie offset, and a second sweep writes the victims with
// ballot prefixes, so the output is in ascending slot order and equal
// scores evict the lower position first ([SNAP] "Tie-breaking").
// Everything is integer: the result is bit-exact for given score bits.
#include <hip/hip_runtime.h>

#include "kvev_device.h"
#include "kvev_kernels.h"

namespace kvev {

namespace {
constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / kWave;
}  // namespace

__global__ __launch_bounds__(kSelThreads) void select_kernel(const SelectArgs P) {
  __shared__ uint32_t hist[256];
  __shared__ uint32_t s_digit, s_rank;
  __shared__ uint32_t w_less[kSelWaves], w_eq[kSelWaves];

  const int u = blockIdx.x;
  const int tid = threadIdx.x;
  const int n = P.seq_len[u];
  if (n < 0 || n > P.max_slots) {  // inconsistent head: flagged, nothing written
    if (tid == 0) P.n_victims[u] = -1;
    return;
  }
  const int m = max(0, n - P.budget);
  const int nc = max(0, n - P.recent);  // candidates: slots [0, nc)
  if (tid == 0) P.n_victims[u] = m;
  if (m == 0) return;
  const float *row = P.score + (size_t)u * P.max_slots;
  int32_t *out = P.victims + (size_t)u * P.max_slots;

  // ---- radix select: key T of rank m (1-based) among the candidates
  uint32_t prefix = 0, pmask = 0, rank = (uint32_t)m;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    if (tid < 256) hist[tid] = 0;
    __syncthreads();
    for (int j = tid; j < nc; j += kSelThreads) {
      const uint32_t k = score_key(row[j]);
      if ((k & pmask) == prefix) atomicAdd(&hist[(k >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid < kWave) {
      // lane l owns digits 4l .. 4l+3
      const uint32_t c0 = hist[4 * tid], c1 = hist[4 * tid + 1], c2 = hist[4 * tid + 2],
                     c3 = hist[4 * tid + 3];
      const uint32_t mine = c0 + c1 + c2 + c3;
      uint32_t incl = mine;
#pragma unroll
      for (int o = 1; o < kWave; o <<= 1) {
        const uint32_t t = __shfl_up(incl, o);
        if (tid >= o) incl += t;
      }
      const uint32_t before = incl - mine;
      if (before < rank && rank <= incl) {  // exactly one lane
        uint32_t r = rank - before, d = 4 * tid;
        if (r > c0) { r -= c0; ++d; if (r > c1) { r -= c1; ++d; if (r > c2) { r -= c2; ++d; } } }
        s_digit = d;
        s_rank = r;
      }
    }
    __syncthreads();
    prefix |= s_digit << shift;
    pmask |= 255u << shift;
    rank = s_rank;
    __syncthreads();
  }
  const uint32_t T = prefix;
  const uint32_t e = rank;  // keys equal to T that are evicted (the lowest slots)

  // ---- emission in ascending slot order
  const int wv = tid / kWave, lane = lane_id();
  const int per = (nc + kSelWaves - 1) / kSelWaves;
  const int c0 = min(nc, wv * per), c1 = min(nc, c0 + per);
  uint32_t nless = 0, neq = 0;
  for (int base = c0; base < c1; base += kWave) {
    const int j = base + lane;
    uint32_t k = 0xffffffffu;
    if (j < c1) k = score_key(row[j]);
    const bool valid = j < c1;
    nless += __popcll(__ballot(valid && k < T));
    neq += __popcll(__ballot(valid && k == T));
  }
  if (lane == 0) {
    w_less[wv] = nless;
    w_eq[wv] = neq;
  }
  __syncthreads();
  uint32_t out_off = 0, eq_off = 0;
  for (int w = 0; w < wv; ++w) {
    const uint32_t taken = eq_off >= e ? 0u : min(w_eq[w], e - eq_off);
    out_off += w_less[w] + taken;
    eq_off += w_eq[w];
  }
  uint32_t eq_seen = eq_off;
  for (int base = c0; base < c1; base += kWave) {
    const int j = base + lane;
    const bool valid = j < c1;
    uint32_t k = 0xffffffffu;
    if (valid) k = score_key(row[j]);
    const bool is_eq = valid && k == T;
    const uint64_t eqm = __ballot(is_eq);
    const uint32_t my_tie = eq_seen + (uint32_t)ballot_prefix(eqm);
    const bool victim = valid && (k < T || (is_eq && my_tie < e));
    const uint64_t vm = __ballot(victim);
    const uint32_t slot_idx = out_off + (uint32_t)ballot_prefix(vm);
    if (victim && slot_idx < (uint32_t)m) out[slot_idx] = j;
    out_off += (uint32_t)__popcll(vm);
    eq_seen += (uint32_t)__popcll(eqm);
  }
}

hipError_t launch_select(const SelectArgs &a, hipStream_t s) {
  hipLaunchKernelGGL(select_kernel, dim3(a.units), dim3(kSelThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace kvev
