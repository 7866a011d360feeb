// hbm_read_probe.hip -- hardware probes (gfx950) that the eviction kernels'
// measurements are read against: the plain HBM read rate (the read ceiling
// of the roofline fractions), how much vector-ALU work overlaps the matrix
// cores, and whether a workgroup barrier waits for outstanding stores.  Not part of the eviction path: they live in their own library,
// libkvev_probe.so, which only the benchmark's probe modes load.
//
// Every pattern reads each byte of a buffer of nbytes (a multiple of 4096)
// exactly once with 16-byte vector loads and folds the words into an xor so
// the loads cannot be dropped; the single store is conditional on a value
// the buffer's contents never produce, so the kernel moves no bytes to HBM.
//   pattern 0  contiguous: grid-stride over 16-byte units, DEPTH loads in
//              flight per lane, consecutive lanes on consecutive units
//   pattern 1  4 KiB blocks through a block list (the paged cache's access
//              shape): each wave takes DEPTH/4 list entries per iteration,
//              one 4 KiB block = four 1 KiB coalesced wave loads
// With the identity list pattern 1 reads the blocks in address order; with
// a shuffled list it reads them in the list's order.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {
constexpr int kThreads = 256;
constexpr int kBlockBytes = 4096;
constexpr int kUnitsPerBlock = kBlockBytes / 16;

template <int DEPTH>
__global__ __launch_bounds__(kThreads) void hbm_read_contiguous(const uint4 *buf, size_t n16,
                                                                uint32_t *sink) {
  const size_t lanes = (size_t)gridDim.x * kThreads;
  uint32_t acc = 0;
  for (size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x; i < n16; i += lanes * DEPTH) {
    uint4 v[DEPTH];
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      const size_t j = i + (size_t)d * lanes;
      v[d] = j < n16 ? buf[j] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) acc ^= v[d].x ^ v[d].y ^ v[d].z ^ v[d].w;
  }
  if (acc == 0xA5A5A5A5u) sink[0] = acc;
}

template <int DEPTH>
__global__ __launch_bounds__(kThreads) void hbm_read_blocks(const uint4 *buf, const int32_t *list,
                                                            int nblk, uint32_t *sink) {
  constexpr int kPerIter = DEPTH / 4;
  const int lane = threadIdx.x & 63;
  const int wave = (blockIdx.x * kThreads + threadIdx.x) >> 6;
  const int waves = (gridDim.x * kThreads) >> 6;
  uint32_t acc = 0;
  for (int b0 = wave * kPerIter; b0 < nblk; b0 += waves * kPerIter) {
    uint4 v[DEPTH];
#pragma unroll
    for (int h = 0; h < kPerIter; ++h) {
      const int e = min(b0 + h, nblk - 1);
      const uint4 *blk = buf + (size_t)list[e] * kUnitsPerBlock;
#pragma unroll
      for (int q = 0; q < 4; ++q) v[h * 4 + q] = blk[q * 64 + lane];
    }
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) acc ^= v[d].x ^ v[d].y ^ v[d].z ^ v[d].w;
  }
  if (acc == 0xA5A5A5A5u) sink[0] = acc;
}

template <int DEPTH>
hipError_t launch(int pattern, const void *buf, size_t nbytes, const int32_t *list, int grid,
                  uint32_t *sink, hipStream_t s) {
  if (pattern == 0)
    hipLaunchKernelGGL(hbm_read_contiguous<DEPTH>, dim3(grid), dim3(kThreads), 0, s,
                       (const uint4 *)buf, nbytes / 16, sink);
  else
    hipLaunchKernelGGL(hbm_read_blocks<DEPTH>, dim3(grid), dim3(kThreads), 0, s,
                       (const uint4 *)buf, list, (int)(nbytes / kBlockBytes), sink);
  return hipGetLastError();
}
}  // namespace

// kvev_probe_read -- one launch of a read pattern over buf.
//   pattern  0 contiguous, 1 4 KiB blocks through `list`
//   depth    16-byte loads in flight per lane: 4, 8 or 16
//   buf      device buffer of nbytes; nbytes a positive multiple of 4096 with
//            nbytes / 4096 < 2^31
//   list     pattern 1: device array of nbytes / 4096 block indices, each in
//            [0, nbytes / 4096) (the caller checks this); unused for pattern 0
//   grid     workgroups of 256 threads, 1 .. 65536
//   sink     device word, written only if the xor of the whole buffer equals
//            0xA5A5A5A5 (the caller fills the buffer so that it does not)
//   stream   hipStream_t, or null for the null stream
// Returns 0, or -1 for a bad argument (nothing launched), or the hipError_t of
// the launch.
extern "C" int kvev_probe_read(int pattern, int depth, const void *buf, size_t nbytes,
                               const int32_t *list, int grid, uint32_t *sink, void *stream) {
  if (pattern < 0 || pattern > 1 || !buf || !sink || nbytes == 0 || nbytes % kBlockBytes ||
      nbytes / kBlockBytes >= (size_t)INT32_MAX || grid < 1 || grid > 65536 ||
      (pattern == 1 && !list))
    return -1;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e;
  switch (depth) {
    case 4: e = launch<4>(pattern, buf, nbytes, list, grid, sink, s); break;
    case 8: e = launch<8>(pattern, buf, nbytes, list, grid, sink, s); break;
    case 16: e = launch<16>(pattern, buf, nbytes, list, grid, sink, s); break;
    default: return -1;
  }
  return (int)e;
}

// ---- MFMA / VALU overlap.  Every thread of a 512-thread workgroup (8 waves,
// two per SIMD) runs `iters` iterations; per iteration a wave does, by mode:
//   0  8 v_mfma_f32_16x16x32_bf16 on 8 independent accumulators
//   1  32 fp32 FMAs on 16 independent chains
//   2  both of the above in the same wave
//   3  the MFMAs on even waves, the FMAs on odd waves
//   4  16 exp2 (with a multiply each) on 16 chains
//   5  the MFMAs and the exp2 chains in the same wave
// Each thread writes one float of `out` (grid * 512 floats), its own index.
namespace {
typedef float ofloatx4 __attribute__((ext_vector_type(4)));
typedef short obf16x8 __attribute__((ext_vector_type(8)));

template <int MODE>
__global__ __launch_bounds__(512) void mfma_valu_overlap(int iters, float seed, float *out) {
  const int tid = threadIdx.x, wv = tid >> 6;
  obf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (short)(0x3f80 + (tid & 7) + i);
    b[i] = (short)(0x3f80 + i);
  }
  ofloatx4 acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = ofloatx4{0.f, 0.f, 0.f, 0.f};
  float v[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) v[i] = seed * (float)(tid + i);
  const bool do_mfma = MODE == 0 || MODE == 2 || MODE == 5 || (MODE == 3 && (wv & 1) == 0);
  const bool do_fma = MODE == 1 || MODE == 2 || (MODE == 3 && (wv & 1) == 1);
  const bool do_exp = MODE == 4 || MODE == 5;
  for (int it = 0; it < iters; ++it) {
    if (do_mfma) {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[i], 0, 0, 0);
    }
    if (do_fma) {
#pragma unroll
      for (int r = 0; r < 2; ++r)
#pragma unroll
        for (int i = 0; i < 16; ++i) v[i] = fmaf(v[i], 0.999f, 0.001f);
    }
    if (do_exp) {
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = __builtin_amdgcn_exp2f(v[i]) * 0.5f;
    }
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) s += acc[i][0] + acc[i][1] + acc[i][2] + acc[i][3];
#pragma unroll
  for (int i = 0; i < 16; ++i) s += v[i];
  out[(size_t)blockIdx.x * 512 + tid] = s;
}
}  // namespace

// kvev_probe_overlap -- one launch of overlap mode `mode` (0..5, above) with
// `grid` workgroups (1 .. 65536) of 512 threads and `iters` (1 .. 2^24)
// iterations; out: device array of grid * 512 floats.  Returns 0, -1 for a
// bad argument (nothing launched), or the hipError_t of the launch.
extern "C" int kvev_probe_overlap(int mode, int grid, int iters, float *out, void *stream) {
  if (mode < 0 || mode > 5 || grid < 1 || grid > 65536 || iters < 1 || iters > (1 << 24) || !out)
    return -1;
  hipStream_t s = (hipStream_t)stream;
  const dim3 g(grid), t(512);
  switch (mode) {
    case 0: hipLaunchKernelGGL(mfma_valu_overlap<0>, g, t, 0, s, iters, 1e-3f, out); break;
    case 1: hipLaunchKernelGGL(mfma_valu_overlap<1>, g, t, 0, s, iters, 1e-3f, out); break;
    case 2: hipLaunchKernelGGL(mfma_valu_overlap<2>, g, t, 0, s, iters, 1e-3f, out); break;
    case 3: hipLaunchKernelGGL(mfma_valu_overlap<3>, g, t, 0, s, iters, 1e-3f, out); break;
    case 4: hipLaunchKernelGGL(mfma_valu_overlap<4>, g, t, 0, s, iters, 1e-3f, out); break;
    default: hipLaunchKernelGGL(mfma_valu_overlap<5>, g, t, 0, s, iters, 1e-3f, out); break;
  }
  return (int)hipGetLastError();
}

// ---- does a workgroup barrier wait for the waves' outstanding global
// stores?  1024-thread workgroups run `iters` rounds of an LDS exchange
// between two barriers; by mode, each thread first issues nothing (0), one
// nontemporal store of its own float of `out` (1), or that store and an
// explicit wait for it (2).  out: grid * 1024 floats, one per thread.
namespace {
template <int MODE>
__global__ __launch_bounds__(1024) void store_barrier(float *out, int iters) {
  __shared__ float s[1024];
  float acc = (float)threadIdx.x;
  float *o = out + (size_t)blockIdx.x * 1024 + threadIdx.x;
  for (int it = 0; it < iters; ++it) {
    if (MODE >= 1) __builtin_nontemporal_store(acc, o);
    if (MODE == 2) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    s[threadIdx.x] = acc;
    __syncthreads();
    acc += s[(threadIdx.x + 1) & 1023];
    __syncthreads();
  }
  if (acc == 12345.f) o[0] = acc;
}
}  // namespace

// kvev_probe_barrier -- one launch of barrier mode `mode` (0..2, above) with
// `grid` (1 .. 65536) workgroups and `iters` (1 .. 2^24) rounds; out: device
// array of grid * 1024 floats.  Returns 0, -1 for a bad argument (nothing
// launched), or the hipError_t of the launch.
extern "C" int kvev_probe_barrier(int mode, int grid, int iters, float *out, void *stream) {
  if (mode < 0 || mode > 2 || grid < 1 || grid > 65536 || iters < 1 || iters > (1 << 24) || !out)
    return -1;
  hipStream_t s = (hipStream_t)stream;
  const dim3 g(grid), t(1024);
  if (mode == 0) hipLaunchKernelGGL(store_barrier<0>, g, t, 0, s, out, iters);
  else if (mode == 1) hipLaunchKernelGGL(store_barrier<1>, g, t, 0, s, out, iters);
  else hipLaunchKernelGGL(store_barrier<2>, g, t, 0, s, out, iters);
  return (int)hipGetLastError();
}
