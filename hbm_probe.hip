// Streaming-read probe: the practical HBM read rate of the device, the
// reference point for the decode kernel's roofline.  Measurement tooling of
// the benchmark, not part of the attention library: `python bench.py
// --build-probe` compiles it into _build/libhbm_probe.so, and `python bench.py
// --read-ceiling` calls it.
//
// Each lane reads 16-byte words, `unroll` of them in flight, grid-stride over
// the buffer, and XOR-folds them so no load can be dropped; a lane writes the
// sink only if the fold equals a value the caller never stores, so the kernel
// writes (almost) nothing.  The loads carry the non-temporal hint or not.
#include <hip/hip_runtime.h>
#include <stddef.h>

typedef unsigned int probe_u32x4 __attribute__((ext_vector_type(4)));

template <int UNROLL, bool NT>
__global__ __launch_bounds__(256) void read_kernel(const probe_u32x4* __restrict__ p, size_t n,
                                                   unsigned* __restrict__ sink) {
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  probe_u32x4 acc = {0u, 0u, 0u, 0u};
  for (; i + (size_t)(UNROLL - 1) * stride < n; i += (size_t)UNROLL * stride) {
    probe_u32x4 v[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u)
      v[u] = NT ? __builtin_nontemporal_load(p + i + (size_t)u * stride) : p[i + (size_t)u * stride];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) acc ^= v[u];
  }
  for (; i < n; i += stride) acc ^= p[i];
  if ((acc.x ^ acc.y ^ acc.z ^ acc.w) == 0x9E3779B9u) sink[0] = 1u;
}

// Reads `bytes` (a positive multiple of 16) from device buffer `buf` once.
// blocks: grid size in 256-lane workgroups (1..1<<20); unroll: 4 or 8 loads in
// flight per lane; nt: 1 for non-temporal loads; sink: one device word.
// Returns 0, -1 on bad arguments, or -5 if the launch failed.
extern "C" int hbm_read_probe(const void* buf, size_t bytes, int blocks, int unroll, int nt,
                              unsigned* sink, void* stream) {
  if (!buf || !sink || bytes == 0 || bytes % 16 != 0 || blocks < 1 || blocks > (1 << 20))
    return -1;
  const size_t n = bytes / 16;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const probe_u32x4* p = static_cast<const probe_u32x4*>(buf);
  if (unroll == 4 && !nt)
    hipLaunchKernelGGL((read_kernel<4, false>), dim3(blocks), dim3(256), 0, s, p, n, sink);
  else if (unroll == 8 && !nt)
    hipLaunchKernelGGL((read_kernel<8, false>), dim3(blocks), dim3(256), 0, s, p, n, sink);
  else if (unroll == 4 && nt)
    hipLaunchKernelGGL((read_kernel<4, true>), dim3(blocks), dim3(256), 0, s, p, n, sink);
  else if (unroll == 8 && nt)
    hipLaunchKernelGGL((read_kernel<8, true>), dim3(blocks), dim3(256), 0, s, p, n, sink);
  else
    return -1;
  return hipGetLastError() == hipSuccess ? 0 : -5;
}
