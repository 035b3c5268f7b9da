// Dispatch scatter on gfx950: every routed (token, expert) entry receives
// the token's row, as bf16 or as FP8 E4M3 codes with per-128-channel
// scales.
//
// "DeepEP" deep dive (llm-infra-atlas, moe/06_deepep): sec. 1.1 (normal
// mode, contiguous per-expert layout, FP8 dispatch), sec. 1.2 (low-latency
// packed masked layout; fp32 or power-of-two scales, column-major), sec. 4.6
// (these kernels move bytes and do no matrix math: HBM is the roof).
//
// Work split: one block per token, one wavefront per piece of the row, so
// the whole row is in flight at once.  Each wave reads its piece once into
// registers (16-byte loads, fully coalesced), quantises it once if asked,
// and stores it to each of the token's K rows with 16-byte stores.  The
// source row is read once, not K times.  (Measured on MI355X at hidden
// 7168: plain stores beat non-temporal ones for this scatter; the kernel
// sits at the chip's write-dominated bandwidth.)
#include "ep_device.hpp"
#include "ep_internal.hpp"
#include "quant.hpp"

namespace ep {

// Row split: one block per token, one wavefront per row piece of NV
// 16-byte vectors per lane (the whole row in flight at once; each wave's
// store instructions write 64 x 16 contiguous bytes).
struct RowSplit {
  int nv;     // vectors per lane
  int waves;  // wavefronts per block (row pieces)
};

inline RowSplit row_split(int vectors, int prefer_nv) {
  RowSplit r;
  r.nv = prefer_nv;
  while ((vectors + kWave * r.nv - 1) / (kWave * r.nv) > 16) ++r.nv;
  r.waves = (vectors + kWave * r.nv - 1) / (kWave * r.nv);
  return r;
}

template <int NV>
__global__ __launch_bounds__(1024) void dispatch_copy(const u32x4* __restrict__ x,
                                                      const int32_t* __restrict__ send_pos,
                                                      u32x4* __restrict__ recv, int V, int K,
                                                      int64_t cap, int32_t* err) {
  const int lane = threadIdx.x & 63;
  const int tok = blockIdx.x;
  const int base = uniform(threadIdx.x >> 6) * kWave * NV;
  const u32x4* src = x + (int64_t)tok * V;
  u32x4 v[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) v[i] = src[min(base + lane + kWave * i, V - 1)];  // in bounds
  const int myrow = lane < K ? send_pos[(int64_t)tok * K + lane] : -1;
  for (int k = 0; k < K; ++k) {
    const int row = __builtin_amdgcn_readlane(myrow, k);
    if (row < 0) continue;
    if (row >= cap) {
      if (lane == 0 && base == 0) set_err(err, EP_DEVERR_CAPACITY);
      continue;
    }
    u32x4* dst = recv + (int64_t)row * V;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int j = base + lane + kWave * i;
      if (j < V) dst[j] = v[i];
    }
  }
}

// P = 16-channel pairs per row (H / 16); a group of 128 channels is 8
// pairs = 8 consecutive lanes, reduced with DPP.
template <int NP, int Q, bool LL>
__global__ __launch_bounds__(NP >= 3 ? 512 : 1024) void dispatch_fp8(const u32x4* __restrict__ x,
                                                     const int32_t* __restrict__ send_pos,
                                                     u32x4* __restrict__ codes,
                                                     void* __restrict__ scales, int P, int K,
                                                     int64_t cap, int G, int RT, int32_t* err) {
  const int lane = threadIdx.x & 63;
  const int tok = blockIdx.x;
  const int base = uniform(threadIdx.x >> 6) * kWave * NP;
  const u32x4* src = x + (int64_t)tok * (2 * (int64_t)P);
  u32x4 lo[NP], hi[NP];
  load_pairs<NP>(src, base, P, lo, hi);
  u32x4 cv[NP];
  float scf[NP];
  uint32_t sce[NP];
#pragma unroll
  for (int i = 0; i < NP; ++i) quantise_pair<Q>(lo[i], hi[i], cv[i], scf[i], sce[i]);
  const int myrow = lane < K ? send_pos[(int64_t)tok * K + lane] : -1;
  for (int k = 0; k < K; ++k) {
    const int row = __builtin_amdgcn_readlane(myrow, k);
    if (row < 0) continue;
    if (row >= cap) {
      if (lane == 0 && base == 0) set_err(err, EP_DEVERR_CAPACITY);
      continue;
    }
    u32x4* dst = codes + (int64_t)row * P;
    int64_t sbase, sstride;
    if (LL) {
      const int e = row / RT, pos = row - e * RT;
      sbase = (int64_t)e * G * RT + pos;
      sstride = RT;
    } else {
      sbase = row;
      sstride = cap;
    }
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int j = base + lane + kWave * i;
      if (j < P) {
        dst[j] = cv[i];
        if ((lane & 7) == 0) {
          const int64_t si = sbase + (int64_t)(j >> 3) * sstride;
          if (Q == EP_QUANT_FP8_F32)
            ((float*)scales)[si] = scf[i];
          else
            ((uint8_t*)scales)[si] = (uint8_t)sce[i];
        }
      }
    }
  }
}

template <int NV>
static void launch_copy_nv(const DispatchArgs& a, int V, int waves, hipStream_t st) {
  const int N = a.g.R * a.g.T;
  hipLaunchKernelGGL(dispatch_copy<NV>, dim3(N), dim3(kWave * waves), 0, st, (const u32x4*)a.x,
                     a.send_pos, (u32x4*)a.recv_x, V, a.g.K, a.cap, a.err);
}

template <int NP, int Q, bool LL>
static void launch_fp8_np(const DispatchArgs& a, int P, int waves, hipStream_t st) {
  const int N = a.g.R * a.g.T;
  hipLaunchKernelGGL((dispatch_fp8<NP, Q, LL>), dim3(N), dim3(kWave * waves), 0, st,
                     (const u32x4*)a.x, a.send_pos, (u32x4*)a.recv_x, a.recv_scales, P, a.g.K,
                     a.cap, a.g.G, a.g.R * a.g.T, a.err);
}

template <int Q, bool LL>
static void launch_fp8_q(const DispatchArgs& a, hipStream_t st) {
  const int P = a.g.H / 16;
  RowSplit rs = row_split(P, 1);
  if (rs.nv >= 3) rs = RowSplit{4, (P + kWave * 4 - 1) / (kWave * 4)};  // <= 8 waves
  switch (rs.nv) {
    case 1: launch_fp8_np<1, Q, LL>(a, P, rs.waves, st); break;
    case 2: launch_fp8_np<2, Q, LL>(a, P, rs.waves, st); break;
    case 3: launch_fp8_np<3, Q, LL>(a, P, rs.waves, st); break;
    default: launch_fp8_np<4, Q, LL>(a, P, rs.waves, st); break;  // hidden <= 32768
  }
}

hipError_t launch_dispatch(const DispatchArgs& a, hipStream_t st) {
  const int64_t N = (int64_t)a.g.R * a.g.T;
  if (N == 0) return hipSuccess;
  if (a.quant == EP_QUANT_NONE) {
    const int V = a.g.H / 8;
    const RowSplit rs = row_split(V, 2);
    switch (rs.nv) {
      case 2: launch_copy_nv<2>(a, V, rs.waves, st); break;
      case 3: launch_copy_nv<3>(a, V, rs.waves, st); break;
      default: launch_copy_nv<4>(a, V, rs.waves, st); break;  // hidden <= 32768
    }
  } else {
    const bool ll = a.mode == EP_MODE_LOW_LATENCY;
    if (a.quant == EP_QUANT_FP8_F32) {
      if (ll) launch_fp8_q<EP_QUANT_FP8_F32, true>(a, st);
      else launch_fp8_q<EP_QUANT_FP8_F32, false>(a, st);
    } else {
      if (ll) launch_fp8_q<EP_QUANT_FP8_UE8M0, true>(a, st);
      else launch_fp8_q<EP_QUANT_FP8_UE8M0, false>(a, st);
    }
  }
  return hipGetLastError();
}

}  // namespace ep
