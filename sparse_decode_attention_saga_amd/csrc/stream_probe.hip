// Streaming-read probe (libsaga_probe.so): the HBM read ceiling the decode kernels are
// measured against. Not part of the decode library's interface; the benchmark loads it.
//
// saga_probe_stream_read reads `bytes` bytes (a multiple of 16) from device memory
// with 16-byte loads: block b reads the b-th of `blocks` contiguous ranges, its
// threads keeping kLoads consecutive 1 KiB-per-wave loads in flight, and writes one
// float per block to `sink` (so the loads are not elided; `sink` holds `blocks`
// floats). `blocks` = 0 picks 1024.
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace {

constexpr int kThreads = 256;
constexpr int kLoads = 8;

__global__ __launch_bounds__(kThreads) void k_stream_read(const uint4* __restrict__ p, size_t n16, size_t per_block,
                                                          float* sink) {
  const size_t base = (size_t)blockIdx.x * per_block;
  const size_t end = base + per_block < n16 ? base + per_block : n16;
  uint32_t acc = 0;
  for (size_t i = base + threadIdx.x; i < end; i += kLoads * kThreads) {
    uint4 v[kLoads];
#pragma unroll
    for (int u = 0; u < kLoads; ++u) {
      const size_t at = i + (size_t)u * kThreads;
      v[u] = at < end ? p[at] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < kLoads; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  __shared__ uint32_t s[kThreads];
  s[threadIdx.x] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = 0;
    for (int t = 0; t < kThreads; ++t) r ^= s[t];
    sink[blockIdx.x] = __uint_as_float(r & 0x007fffffu);  // a finite value
  }
}

}  // namespace

extern "C" int saga_probe_stream_read(const void* p, size_t bytes, float* sink, int blocks, void* stream) {
  if (!p || !sink || bytes % 16 != 0 || blocks < 0) return 1;
  if (blocks == 0) blocks = 1024;
  const size_t n16 = bytes / 16;
  const size_t per_block = (n16 + blocks - 1) / blocks;
  (void)hipGetLastError();
  hipLaunchKernelGGL(k_stream_read, dim3(blocks), dim3(kThreads), 0, (hipStream_t)stream,
                     reinterpret_cast<const uint4*>(p), n16, per_block, sink);
  return hipGetLastError() == hipSuccess ? 0 : 5;
}
