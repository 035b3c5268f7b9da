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

// Fan-out: each of `rows` source rows (V vectors) is read once and written to
// `copies` rows, row k * rows + t (`copies` contiguous destination segments):
// the bf16 dispatch's read/write mix with the simplest addresses.  One block
// per source row: 4 waves holding the row in registers (PER = 4 vectors per
// lane), or 14 waves of one vector each that wait for one copy's stores
// before the next (PACE).
template <int PER, bool PACE>
__global__ __launch_bounds__(1024) void probe_fanout(const u32x4* __restrict__ src,
                                                     u32x4* __restrict__ dst, int V, int rows,
                                                     int copies) {
  const int t = blockIdx.x;
  u32x4 v[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int j = threadIdx.x + i * blockDim.x;
    v[i] = j < V ? src[(int64_t)t * V + j] : u32x4{0u, 0u, 0u, 0u};
  }
  for (int k = 0; k < copies; ++k) {
    u32x4* d = dst + ((int64_t)k * rows + t) * V;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int j = threadIdx.x + i * blockDim.x;
      if (j < V) d[j] = v[i];
    }
    // s_waitcnt immediate (gfx9 family): vmcnt(0) only (expcnt 7, lgkmcnt 15)
    if (PACE) __builtin_amdgcn_s_waitcnt(0x0F70);
  }
}

// Fan-in: each of `rows` destination rows is the xor of `copies` source rows,
// row k * rows + t: the bf16 combine's read/write mix with the simplest
// addresses.  One block per destination row, PER vectors per lane;
// non-temporal loads and stores, as in the combine.
template <int PER>
__global__ __launch_bounds__(1024) void probe_fanin(const u32x4* __restrict__ src,
                                                    u32x4* __restrict__ dst, int V, int rows,
                                                    int copies) {
  const int t = blockIdx.x;
  u32x4 acc[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) acc[i] = u32x4{0u, 0u, 0u, 0u};
  for (int k = 0; k < copies; ++k) {
    const u32x4* s = src + ((int64_t)k * rows + t) * V;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int j = threadIdx.x + i * blockDim.x;
      if (j < V) acc[i] ^= __builtin_nontemporal_load(s + j);
    }
  }
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int j = threadIdx.x + i * blockDim.x;
    if (j < V) __builtin_nontemporal_store(acc[i], dst + (int64_t)t * V + j);
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

// Fan-out probe (probe_fanout): src holds rows x row_vectors 16-byte vectors,
// dst rows x copies x row_vectors.  form 0: four waves, four vectors per lane
// (row_vectors <= 1024); form 1: one vector per lane, waves paced per copy
// (row_vectors a multiple of 64, at most 1024).  Returns 0, or -1 for a bad
// argument or launch error.
extern "C" int bench_fanout_launch(const void* src, void* dst, int64_t row_vectors, int64_t rows,
                                   int copies, int form, void* stream) {
  if (!src || !dst || row_vectors < 1 || row_vectors > 1024 || rows < 1 || rows > (1 << 30) ||
      copies < 1 || copies > 64)
    return -1;
  hipStream_t s = (hipStream_t)stream;
  const int V = (int)row_vectors, n = (int)rows;
  if (form == 0) {
    hipLaunchKernelGGL((probe_fanout<4, false>), dim3(n), dim3(256), 0, s, (const u32x4*)src,
                       (u32x4*)dst, V, n, copies);
  } else if (form == 1) {
    if (V % 64 != 0) return -1;
    hipLaunchKernelGGL((probe_fanout<1, true>), dim3(n), dim3(V), 0, s, (const u32x4*)src,
                       (u32x4*)dst, V, n, copies);
  } else {
    return -1;
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// Fan-in probe (probe_fanin): src holds copies x rows x row_vectors 16-byte
// vectors, dst rows x row_vectors.  form 0: one vector per lane (row_vectors
// a multiple of 64, at most 1024); form 1: four waves, four vectors per lane
// (row_vectors <= 1024).  Returns 0, or -1 for a bad argument or launch
// error.
extern "C" int bench_fanin_launch(const void* src, void* dst, int64_t row_vectors, int64_t rows,
                                  int copies, int form, void* stream) {
  if (!src || !dst || row_vectors < 1 || row_vectors > 1024 || rows < 1 || rows > (1 << 30) ||
      copies < 1 || copies > 64)
    return -1;
  hipStream_t s = (hipStream_t)stream;
  const int V = (int)row_vectors, n = (int)rows;
  if (form == 0) {
    if (V % 64 != 0) return -1;
    hipLaunchKernelGGL((probe_fanin<1>), dim3(n), dim3(V), 0, s, (const u32x4*)src,
                       (u32x4*)dst, V, n, copies);
  } else if (form == 1) {
    hipLaunchKernelGGL((probe_fanin<4>), dim3(n), dim3(256), 0, s, (const u32x4*)src,
                       (u32x4*)dst, V, n, copies);
  } else {
    return -1;
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}
