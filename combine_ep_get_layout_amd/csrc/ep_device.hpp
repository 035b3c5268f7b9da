// Device-side helpers shared by the libep kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/ep.h"

namespace ep {

constexpr int kWave = 64;

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// popcount(mask & lanes-below-me) via the mbcnt pair
__device__ __forceinline__ int rank_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

__device__ __forceinline__ uint64_t lanes_below() {
  const int l = lane_id();
  return l == 0 ? 0ull : (~0ull >> (64 - l));
}

// Lanes of `valid` whose `key` equals this lane's, found with one ballot per
// key bit (a wave-wide multi-split without LDS or atomics).  Every lane of
// the wave must call it; the result for a lane outside `valid` is garbage.
__device__ __forceinline__ uint64_t match_key(uint32_t key, int nbits, uint64_t valid) {
  uint64_t m = valid;
  for (int b = 0; b < nbits; ++b) {
    const bool bit = (key >> b) & 1u;
    const uint64_t ones = __ballot(bit);
    m &= bit ? ones : ~ones;
  }
  return m;
}

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Hand-off point for LDS data one lane of a wavefront stores and other
// lanes of the same wavefront load afterwards.  The LDS unit executes one
// wavefront's operations in issue order, so the only hazard is the compiler
// moving an access across the hand-off; the wavefront-scope fences (no
// instructions) and the wave barrier forbid that.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Work-groups are dealt to the kXcds dies round-robin (block b on die
// b % kXcds), and each die has its own L2.  xcd_run maps block b to item
// (b % kXcds) * per + b / kXcds, per = ceil(n / kXcds): each die walks a
// contiguous run of items in order.  A grid of xcd_blocks(n) = kXcds * per
// blocks covers every item once (items >= n exit).
constexpr int kXcds = 8;

__host__ __device__ __forceinline__ int xcd_blocks(int n) {
  return kXcds * ((n + kXcds - 1) / kXcds);
}

__device__ __forceinline__ int xcd_run(int b, int n) {
  const int per = (n + kXcds - 1) / kXcds;
  return (b % kXcds) * per + b / kXcds;
}

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> OCP E4M3 (no infinities, max 448) by integer rounding of the
// binary32 pattern: keep 3 mantissa bits with round-to-nearest-even, rebias
// the exponent from 127 to 7; magnitudes below 2^-6 are subnormal
// multiples of 2^-9 (rounded with v_rndne); magnitudes above 448 saturate.
__device__ __forceinline__ uint32_t f32_to_e4m3(float f) {
  const uint32_t u = __float_as_uint(f);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7FFFFFFFu;
  uint32_t mag;
  if (a > 0x43E00000u) {            // > 448
    mag = 0x7Eu;
  } else if (a < 0x3C800000u) {     // < 2^-6
    mag = (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f);
  } else {
    mag = ((a + 0x7FFFFu + ((a >> 20) & 1u)) >> 20) - (120u << 3);
  }
  return sign | mag;
}

// max over groups of 8 consecutive lanes (DPP: quad swaps, then half-row mirror)
__device__ __forceinline__ uint32_t max8_lanes(uint32_t v) {
  uint32_t t;
  t = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false);  // quad_perm 1,0,3,2
  v = v > t ? v : t;
  t = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false);  // quad_perm 2,3,0,1
  v = v > t ? v : t;
  t = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false); // row_half_mirror
  v = v > t ? v : t;
  return v;
}

__device__ __forceinline__ void set_err(int32_t* err, int bits) {
  if (err) atomicOr(err, bits);
}

template <typename T>
__device__ __forceinline__ void st_nt(T* p, const T& v) {
  __builtin_nontemporal_store(v, p);
}

__device__ __forceinline__ void st_nt16(uint4* p, const uint4& v) {
  __builtin_nontemporal_store(v.x, &p->x);
  __builtin_nontemporal_store(v.y, &p->y);
  __builtin_nontemporal_store(v.z, &p->z);
  __builtin_nontemporal_store(v.w, &p->w);
}

}  // namespace ep
