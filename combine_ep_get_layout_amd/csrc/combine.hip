// Combine gather-reduce on gfx950: each token gathers the expert outputs of
// its K routed rows and takes their top-k weighted sum, fp32 accumulation in
// k order (fused multiply-add), rounded to bf16 nearest-even.
//
// "DeepEP" deep dive (llm-infra-atlas, moe/06_deepep), sec. 2.3: combine
// walks dispatch's address book backwards; sec. 5: combine is the inverse
// of dispatch; sec. 1.1: bf16 combine.
//
// Work split: one wavefront owns one piece of one output row.  The K row
// indices and weights are loaded once per wave (one lane each) and read as
// scalars; each k streams one piece of one receive row with 16-byte loads.
#include "ep_device.hpp"
#include "ep_internal.hpp"

namespace ep {

constexpr int kCombineWaves = 4;

// Grid: x = token / 4 (one wavefront per token), y = row piece.
template <int NV>
__global__ __launch_bounds__(256) void combine_rows(const u32x4* __restrict__ y,
                                                    const int32_t* __restrict__ send_pos,
                                                    const float* __restrict__ w,
                                                    u32x4* __restrict__ out, int V, int K,
                                                    int n_tok, int64_t y_rows, int32_t* err) {
  const int lane = threadIdx.x & 63;
  const int tok = uniform(blockIdx.x * kCombineWaves + (threadIdx.x >> 6));
  if (tok >= n_tok) return;
  const int base = blockIdx.y * kWave * NV;
  const int myrow = lane < K ? send_pos[(int64_t)tok * K + lane] : -1;
  const float myw = lane < K ? w[(int64_t)tok * K + lane] : 0.0f;
  float acc[NV][8];
#pragma unroll
  for (int i = 0; i < NV; ++i)
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[i][q] = 0.0f;
  for (int k = 0; k < K; ++k) {
    const int row = __builtin_amdgcn_readlane(myrow, k);
    if (row < 0) continue;
    if (row >= y_rows) {
      if (lane == 0 && base == 0) set_err(err, EP_DEVERR_CAPACITY);
      continue;
    }
    const float wk = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(myw), k));
    const u32x4* src = y + (int64_t)row * V;
    u32x4 v[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {  // clamped, so every load is in bounds
      const int j = min(base + lane + kWave * i, V - 1);
      v[i] = __builtin_nontemporal_load(src + j);
    }
#pragma unroll
    for (int i = 0; i < NV; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[i][2 * q] = __builtin_fmaf(wk, bf16_lo(v[i][q]), acc[i][2 * q]);
        acc[i][2 * q + 1] = __builtin_fmaf(wk, bf16_hi(v[i][q]), acc[i][2 * q + 1]);
      }
  }
  u32x4* dst = out + (int64_t)tok * V;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int j = base + lane + kWave * i;
    if (j < V) {
      u32x4 o;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        o[q] = f32_to_bf16_rne(acc[i][2 * q]) | (f32_to_bf16_rne(acc[i][2 * q + 1]) << 16);
      __builtin_nontemporal_store(o, dst + j);
    }
  }
}

template <int NV>
static void launch_nv(const CombineArgs& a, int V, int npieces, hipStream_t st) {
  const int N = a.g.R * a.g.T;
  const int blocks = (N + kCombineWaves - 1) / kCombineWaves;
  hipLaunchKernelGGL(combine_rows<NV>, dim3(blocks, npieces), dim3(256), 0, st,
                     (const u32x4*)a.y, a.send_pos, a.w, (u32x4*)a.out, V, a.g.K, N, a.y_rows,
                     a.err);
}

hipError_t launch_combine(const CombineArgs& a, hipStream_t st) {
  const int64_t N = (int64_t)a.g.R * a.g.T;
  if (N == 0) return hipSuccess;
  const int V = a.g.H / 8;
  const int npieces = (V + kWave * 8 - 1) / (kWave * 8);
  const int nv = (V + kWave * npieces - 1) / (kWave * npieces);
  switch (nv) {
    case 1: launch_nv<1>(a, V, npieces, st); break;
    case 2: launch_nv<2>(a, V, npieces, st); break;
    case 3: launch_nv<3>(a, V, npieces, st); break;
    case 4: launch_nv<4>(a, V, npieces, st); break;
    case 5: launch_nv<5>(a, V, npieces, st); break;
    case 6: launch_nv<6>(a, V, npieces, st); break;
    case 7: launch_nv<7>(a, V, npieces, st); break;
    default: launch_nv<8>(a, V, npieces, st); break;
  }
  return hipGetLastError();
}

}  // namespace ep
