// FP8 E4M3 quantisation of bf16 data in 128-channel groups (gfx950).
//
// "DeepEP" deep dive (llm-infra-atlas, moe/06_deepep), sec. 1.1 / 1.2: FP8
// dispatch with one scale per 128 channels; the scale is fp32 (amax / 448,
// 448 being the largest E4M3 value) or a power of two (UE8M0: the fp32
// scale rounded up, stored as its biased exponent).  The amax is floored at
// 1e-4 so an all-zero group has a finite scale.
//
// Data layout: a lane holds one "pair" = 2 x 16 bytes = 16 consecutive bf16
// channels; a 128-channel group is 8 consecutive lanes.
#pragma once

#include "ep_device.hpp"
#include "ep_internal.hpp"

namespace ep {

// |bf16| maximum of 16 channels, as a bf16 bit pattern (non-negative bf16
// patterns order like their values).
__device__ __forceinline__ uint32_t absmax16(const u32x4& a, const u32x4& b) {
  uint32_t m = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t w0 = a[q] & 0x7FFF7FFFu, w1 = b[q] & 0x7FFF7FFFu;
    m = max(m, max(w0 & 0xFFFFu, w0 >> 16));
    m = max(m, max(w1 & 0xFFFFu, w1 >> 16));
  }
  return m;
}

// 8 bf16 channels (one 16-byte vector) -> 8 E4M3 codes in two words.
template <int Q>
__device__ __forceinline__ void encode8(const u32x4& v, float sc, int shift, uint32_t& c0,
                                        uint32_t& c1) {
  uint32_t b[8];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    float f0 = bf16_lo(v[q]), f1 = bf16_hi(v[q]);
    if (Q == EP_QUANT_FP8_F32) {
      f0 = __fdiv_rn(f0, sc);
      f1 = __fdiv_rn(f1, sc);
    } else {
      f0 = __builtin_ldexpf(f0, shift);
      f1 = __builtin_ldexpf(f1, shift);
    }
    b[2 * q] = f32_to_e4m3(f0);
    b[2 * q + 1] = f32_to_e4m3(f1);
  }
  c0 = b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24);
  c1 = b[4] | (b[5] << 8) | (b[6] << 16) | (b[7] << 24);
}

// Load NP pairs per lane (pair j = base + lane + 64*i), clamped so every
// load is in bounds; pairs past the row read as zero.
template <int NP>
__device__ __forceinline__ void load_pairs(const u32x4* src, int base, int P, u32x4 (&lo)[NP],
                                           u32x4 (&hi)[NP]) {
  const int lane = lane_id();
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const int j = base + lane + kWave * i;
    const int jc = min(j, P - 1);
    lo[i] = __builtin_nontemporal_load(src + 2 * jc);
    hi[i] = __builtin_nontemporal_load(src + 2 * jc + 1);
  }
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    if (base + lane + kWave * i >= P) {
      lo[i] = u32x4{0u, 0u, 0u, 0u};
      hi[i] = u32x4{0u, 0u, 0u, 0u};
    }
  }
}

// Quantise one pair; every lane of the wave must call it (the group amax
// is reduced across 8 lanes with DPP).  Out: 16 codes, the fp32 scale and
// the UE8M0 exponent byte (the one that matches Q is meaningful).
template <int Q>
__device__ __forceinline__ void quantise_pair(const u32x4& lo, const u32x4& hi, u32x4& codes,
                                              float& scale_f32, uint32_t& scale_e8) {
  const uint32_t am = max8_lanes(absmax16(lo, hi));
  const float a = fmaxf(__uint_as_float(am << 16), 1e-4f);
  const float r = __fdiv_rn(a, 448.0f);
  int shift = 0;
  scale_f32 = r;
  scale_e8 = 0;
  if (Q == EP_QUANT_FP8_UE8M0) {
    const uint32_t rb = __float_as_uint(r);
    const uint32_t ex = ((rb >> 23) & 0xFFu) + ((rb & 0x7FFFFFu) != 0u ? 1u : 0u);
    scale_e8 = ex;
    shift = 127 - (int)ex;
  }
  uint32_t c0, c1, c2, c3;
  encode8<Q>(lo, r, shift, c0, c1);
  encode8<Q>(hi, r, shift, c2, c3);
  codes = u32x4{c0, c1, c2, c3};
}

}  // namespace ep
