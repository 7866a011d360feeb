// kvev_device.h -- device-side helpers shared by the gfx950 kernels of libkvev.
//
// Types for the CDNA4 matrix instructions, 16-byte vector loads, the
// order-preserving integer key of an fp32 score, and wave-level reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvev {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kBlock = 16;     // tokens per cache block
constexpr int kWave = 64;      // CDNA wavefront size

// log2(e) in fp32: p = exp(x) is evaluated as exp2(x * log2(e)).
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ uint4 ld16(const void *p) { return *reinterpret_cast<const uint4 *>(p); }

// 16 bytes from global memory straight into LDS (global_load_lds_dwordx4):
// lane l's bytes land at lds_wave_base + 16 * l; lds_wave_base must be the
// same for every lane of the wave.  Completion is counted like a load.
__device__ __forceinline__ void ld16_to_lds(const void *g, void *lds_wave_base) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)g,
                                   (__attribute__((address_space(3))) void *)lds_wave_base, 16, 0, 0);
}
__device__ __forceinline__ void st16(void *p, uint4 v) { *reinterpret_cast<uint4 *>(p) = v; }
// 16-byte store with the nontemporal hint (global_store_dwordx4 ... nt): for
// rows written once and not read again soon, so they go out to HBM now
// instead of staying as dirty lines in the Infinity Cache, whose later
// write-back would take bandwidth from whatever streams through next.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void st16_nt(void *p, uint4 v) {
  __builtin_nontemporal_store(__builtin_bit_cast(u32x4_t, v), reinterpret_cast<u32x4_t *>(p));
}

// 16x16 tile, contraction 32, bf16 inputs, fp32 accumulate (v_mfma_f32_16x16x32_bf16).
// A operand: lane l supplies row (l % 16), 8 consecutive contraction slots of
// group (l / 16); B operand: lane l supplies column (l % 16), same slots.
// Result: lane l holds C[(l / 16) * 4 + e][l % 16], e = 0..3.
__device__ __forceinline__ floatx4 mfma_bf16(uint4 a, uint4 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Same tile with fp32 inputs, contraction 4 (v_mfma_f32_16x16x4_f32): one
// contraction slot per lane, group (l / 16).  A uint4 carries four slots,
// consumed by four instructions.
__device__ __forceinline__ floatx4 mfma_f32x4(uint4 a, uint4 b, floatx4 c) {
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.x), __uint_as_float(b.x), c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.y), __uint_as_float(b.y), c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.z), __uint_as_float(b.z), c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.w), __uint_as_float(b.w), c, 0, 0, 0);
  return c;
}

template <bool BF16>
__device__ __forceinline__ floatx4 mfma_unit(uint4 a, uint4 b, floatx4 c) {
  if constexpr (BF16)
    return mfma_bf16(a, b, c);
  else
    return mfma_f32x4(a, b, c);
}

// Sum of squares of the values packed in a uint4 (8 bf16 or 4 fp32), fp32.
template <bool BF16>
__device__ __forceinline__ float sumsq_unit(uint4 v) {
  if constexpr (BF16) {
    float s = 0.f;
    uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float lo = __uint_as_float(w[i] << 16), hi = __uint_as_float(w[i] & 0xffff0000u);
      s = fmaf(lo, lo, s);
      s = fmaf(hi, hi, s);
    }
    return s;
  } else {
    float s = 0.f;
    s = fmaf(__uint_as_float(v.x), __uint_as_float(v.x), s);
    s = fmaf(__uint_as_float(v.y), __uint_as_float(v.y), s);
    s = fmaf(__uint_as_float(v.z), __uint_as_float(v.z), s);
    s = fmaf(__uint_as_float(v.w), __uint_as_float(v.w), s);
    return s;
  }
}

// Order-preserving key of an fp32 score: a < b numerically <=> key(a) < key(b);
// -0 and +0 share a key; every NaN maps above +inf.
__device__ __forceinline__ uint32_t score_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0xffffffffu;  // NaN
  if (u == 0x80000000u) u = 0u;                              // -0 -> +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

// Inclusive prefix sum over the wave's 64 lanes, on DPP lane moves (no LDS
// round trips): shifts by 1, 2, 4 and 8 within each row of 16 lanes, then
// lane 15 of each row added into the next row, and lane 31 into rows 2 and
// 3.  A lane with no source reads 0.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, false);  // row_shr:1
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, false);  // row_shr:2
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, false);  // row_shr:4
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, false);  // row_shr:8
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xa, 0xf, false);  // row_bcast:15
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return v;
}

// Exclusive prefix count of set bits below this lane in a 64-bit ballot.
__device__ __forceinline__ int ballot_prefix(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

}  // namespace kvev
