// HBM bandwidth probes for bench.py (gfx950): plain streaming kernels that
// read only, write only, or copy, with 16-byte vector accesses, so that the
// bench can state the device's measured read and write rates next to the
// method's kernels in the same process.  Each block streams a contiguous
// chunk of the buffer (chunk = n / blocks, rounded to whole blocks of
// vectors); U vectors per thread are in flight per round.  NT selects
// non-temporal loads / stores.  Built by combine_ep_get_layout_amd/build.py
// into libbench_probe.so; not part of libep.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

namespace {

template <bool NT>
__device__ __forceinline__ u32x4 ld(const u32x4* p) {
  return NT ? __builtin_nontemporal_load(p) : *p;
}

template <bool NT>
__device__ __forceinline__ void st(u32x4* p, const u32x4& v) {
  if (NT) __builtin_nontemporal_store(v, p);
  else *p = v;
}

// Reads every vector of its chunk; the xor of the loaded values is stored
// only if it equals a value that does not occur, so the loads stay and the
// probe writes nothing.
template <int U, bool NT>
__global__ __launch_bounds__(256) void probe_read(const u32x4* __restrict__ src, int64_t n,
                                                  int64_t chunk, u32x4* sink) {
  const int64_t lo = (int64_t)blockIdx.x * chunk;
  const int64_t hi = lo + chunk < n ? lo + chunk : n;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (int64_t i = lo + threadIdx.x; i < hi; i += (int64_t)U * blockDim.x) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t j = i + (int64_t)u * blockDim.x;
      v[u] = j < hi ? ld<NT>(src + j) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u];
  }
  if (acc[0] == 0x9E3779B9u && acc[1] == 0x7F4A7C15u && acc[2] == 0x85EBCA6Bu &&
      acc[3] == 0xC2B2AE35u)
    sink[threadIdx.x] = acc;
}

template <int U, bool NT>
__global__ __launch_bounds__(256) void probe_write(u32x4* __restrict__ dst, int64_t n,
                                                   int64_t chunk, uint32_t seed) {
  const int64_t lo = (int64_t)blockIdx.x * chunk;
  const int64_t hi = lo + chunk < n ? lo + chunk : n;
  for (int64_t i = lo + threadIdx.x; i < hi; i += (int64_t)U * blockDim.x) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t j = i + (int64_t)u * blockDim.x;
      if (j < hi) st<NT>(dst + j, u32x4{seed, (uint32_t)j, (uint32_t)(j >> 32), seed ^ 1u});
    }
  }
}

template <int U, bool NT>
__global__ __launch_bounds__(256) void probe_copy(const u32x4* __restrict__ src,
                                                  u32x4* __restrict__ dst, int64_t n,
                                                  int64_t chunk) {
  const int64_t lo = (int64_t)blockIdx.x * chunk;
  const int64_t hi = lo + chunk < n ? lo + chunk : n;
  for (int64_t i = lo + threadIdx.x; i < hi; i += (int64_t)U * blockDim.x) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t j = i + (int64_t)u * blockDim.x;
      v[u] = j < hi ? ld<NT>(src + j) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t j = i + (int64_t)u * blockDim.x;
      if (j < hi) st<NT>(dst + j, v[u]);
    }
  }
}

int64_t chunk_of(int64_t n, int blocks) {
  const int64_t c = (n + blocks - 1) / blocks;
  return (c + 255) / 256 * 256;  // whole rounds of a 256-thread block
}

template <int U, bool NT>
int launch(int kind, const void* src, void* dst, int64_t bytes, int blocks, hipStream_t s) {
  const int64_t n = bytes / 16;
  const int64_t chunk = chunk_of(n, blocks);
  const int nb = (int)((n + chunk - 1) / chunk);
  if (kind == 0)
    hipLaunchKernelGGL((probe_read<U, NT>), dim3(nb), dim3(256), 0, s, (const u32x4*)src, n,
                       chunk, (u32x4*)dst);
  else if (kind == 1)
    hipLaunchKernelGGL((probe_write<U, NT>), dim3(nb), dim3(256), 0, s, (u32x4*)dst, n, chunk,
                       0x5A5A0001u);
  else
    hipLaunchKernelGGL((probe_copy<U, NT>), dim3(nb), dim3(256), 0, s, (const u32x4*)src,
                       (u32x4*)dst, n, chunk);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace

// kind: 0 read-only (dst: a 4 KiB sink that is never written in practice),
// 1 write-only (src unused), 2 copy.  bytes: a multiple of 16; src and dst
// 16-byte aligned device buffers of at least `bytes` (the sink: 4 KiB).
// unroll: 1, 2, 4 or 8 vectors per thread in flight; nt: non-temporal
// accesses; blocks: grid size (chunks).  Returns 0, or -1 for a bad argument
// or launch error.
extern "C" int bench_probe_launch(int kind, const void* src, void* dst, int64_t bytes,
                                  int unroll, int nt, int blocks, void* stream) {
  if (kind < 0 || kind > 2 || bytes <= 0 || bytes % 16 != 0 || blocks < 1) return -1;
  if ((kind != 1 && !src) || !dst) return -1;
  hipStream_t s = (hipStream_t)stream;
  switch (unroll * 2 + (nt ? 1 : 0)) {
    case 2: return launch<1, false>(kind, src, dst, bytes, blocks, s);
    case 3: return launch<1, true>(kind, src, dst, bytes, blocks, s);
    case 4: return launch<2, false>(kind, src, dst, bytes, blocks, s);
    case 5: return launch<2, true>(kind, src, dst, bytes, blocks, s);
    case 8: return launch<4, false>(kind, src, dst, bytes, blocks, s);
    case 9: return launch<4, true>(kind, src, dst, bytes, blocks, s);
    case 16: return launch<8, false>(kind, src, dst, bytes, blocks, s);
    case 17: return launch<8, true>(kind, src, dst, bytes, blocks, s);
    default: return -1;
  }
}
