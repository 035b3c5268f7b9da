// Dispatch scatter on gfx950: every routed (token, expert) entry receives
// the token's row, as bf16 or as FP8 E4M3 codes with per-128-channel
// scales.
//
// "DeepEP" deep dive (llm-infra-atlas, moe/06_deepep): sec. 1.1 (normal
// mode, contiguous per-expert layout, FP8 dispatch), sec. 1.2 (low-latency
// packed masked layout; fp32 or power-of-two scales, column-major), sec. 4.6
// (these kernels move bytes and do no matrix math: HBM is the roof).
//
// Work split: one wavefront owns one piece of one token row (the whole row
// for hidden <= 4096 bf16 channels per 64 lanes x 8 vectors).  It reads the
// piece once into registers (16-byte loads, fully coalesced), quantises it
// once if asked, and stores it to each of the token's K rows (16-byte
// non-temporal stores: the receive buffer is not re-read by this kernel).
// The source row is therefore read once, not K times.
#include "ep_device.hpp"
#include "ep_internal.hpp"
#include "quant.hpp"

namespace ep {

constexpr int kWavesPerBlock = 4;

// Grid: x = token / 4 (one wavefront per token), y = row piece.
template <int NV>
__global__ __launch_bounds__(256) void dispatch_copy(const u32x4* __restrict__ x,
                                                     const int32_t* __restrict__ send_pos,
                                                     u32x4* __restrict__ recv, int V, int K,
                                                     int n_tok, int64_t cap, int32_t* err) {
  const int lane = threadIdx.x & 63;
  const int tok = uniform(blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6));
  if (tok >= n_tok) return;
  const int base = blockIdx.y * kWave * NV;
  const u32x4* src = x + (int64_t)tok * V;
  u32x4 v[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {  // clamped, so every load is in bounds
    const int j = min(base + lane + kWave * i, V - 1);
    v[i] = __builtin_nontemporal_load(src + j);
  }
  const int myrow = lane < K ? send_pos[(int64_t)tok * K + lane] : -1;
  for (int k = 0; k < K; ++k) {
    const int row = __builtin_amdgcn_readlane(myrow, k);
    if (row < 0) continue;
    if (row >= cap) {
      if (lane == 0) set_err(err, EP_DEVERR_CAPACITY);
      continue;
    }
    u32x4* dst = recv + (int64_t)row * V;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int j = base + lane + kWave * i;
      if (j < V) __builtin_nontemporal_store(v[i], dst + j);
    }
  }
}

// P = 16-channel pairs per row (H / 16); a group of 128 channels is 8
// pairs = 8 consecutive lanes, reduced with DPP.
template <int NP, int Q, bool LL>
__global__ __launch_bounds__(256) void dispatch_fp8(const u32x4* __restrict__ x,
                                                    const int32_t* __restrict__ send_pos,
                                                    u32x4* __restrict__ codes,
                                                    void* __restrict__ scales, int P, int K,
                                                    int n_tok, int64_t cap, int G, int RT,
                                                    int32_t* err) {
  const int lane = threadIdx.x & 63;
  const int tok = uniform(blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6));
  if (tok >= n_tok) return;
  const int base = blockIdx.y * kWave * NP;
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
      if (lane == 0) set_err(err, EP_DEVERR_CAPACITY);
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
        __builtin_nontemporal_store(cv[i], dst + j);
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
static void launch_copy_nv(const DispatchArgs& a, int V, int npieces, hipStream_t st) {
  const int N = a.g.R * a.g.T;
  const int blocks = (N + kWavesPerBlock - 1) / kWavesPerBlock;
  hipLaunchKernelGGL(dispatch_copy<NV>, dim3(blocks, npieces), dim3(256), 0, st,
                     (const u32x4*)a.x, a.send_pos, (u32x4*)a.recv_x, V, a.g.K, N, a.cap, a.err);
}

template <int NP, int Q, bool LL>
static void launch_fp8_np(const DispatchArgs& a, int P, int npieces, hipStream_t st) {
  const int N = a.g.R * a.g.T;
  const int blocks = (N + kWavesPerBlock - 1) / kWavesPerBlock;
  hipLaunchKernelGGL((dispatch_fp8<NP, Q, LL>), dim3(blocks, npieces), dim3(256), 0, st,
                     (const u32x4*)a.x, a.send_pos, (u32x4*)a.recv_x, a.recv_scales, P, a.g.K, N,
                     a.cap, a.g.G, a.g.R * a.g.T, a.err);
}

template <int Q, bool LL>
static void launch_fp8_q(const DispatchArgs& a, hipStream_t st) {
  const int P = a.g.H / 16;
  const int npieces = (P + kWave * 8 - 1) / (kWave * 8);
  const int np = (P + kWave * npieces - 1) / (kWave * npieces);
  switch (np) {
    case 1: launch_fp8_np<1, Q, LL>(a, P, npieces, st); break;
    case 2: launch_fp8_np<2, Q, LL>(a, P, npieces, st); break;
    case 3: launch_fp8_np<3, Q, LL>(a, P, npieces, st); break;
    case 4: launch_fp8_np<4, Q, LL>(a, P, npieces, st); break;
    case 5: launch_fp8_np<5, Q, LL>(a, P, npieces, st); break;
    case 6: launch_fp8_np<6, Q, LL>(a, P, npieces, st); break;
    case 7: launch_fp8_np<7, Q, LL>(a, P, npieces, st); break;
    default: launch_fp8_np<8, Q, LL>(a, P, npieces, st); break;
  }
}

hipError_t launch_dispatch(const DispatchArgs& a, hipStream_t st) {
  const int64_t N = (int64_t)a.g.R * a.g.T;
  if (N == 0) return hipSuccess;
  if (a.quant == EP_QUANT_NONE) {
    const int V = a.g.H / 8;
    const int npieces = (V + kWave * 8 - 1) / (kWave * 8);
    const int nv = (V + kWave * npieces - 1) / (kWave * npieces);
    switch (nv) {
      case 1: launch_copy_nv<1>(a, V, npieces, st); break;
      case 2: launch_copy_nv<2>(a, V, npieces, st); break;
      case 3: launch_copy_nv<3>(a, V, npieces, st); break;
      case 4: launch_copy_nv<4>(a, V, npieces, st); break;
      case 5: launch_copy_nv<5>(a, V, npieces, st); break;
      case 6: launch_copy_nv<6>(a, V, npieces, st); break;
      case 7: launch_copy_nv<7>(a, V, npieces, st); break;
      default: launch_copy_nv<8>(a, V, npieces, st); break;
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
