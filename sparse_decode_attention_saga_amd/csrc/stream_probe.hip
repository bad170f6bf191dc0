// Streaming-read probe (libsaga_probe.so): the HBM read ceiling the decode kernels are
// measured against. Not part of the decode library's interface; the benchmark loads it.
//
// saga_probe_stream_read reads `bytes` bytes (a multiple of 16) from device memory
// with 16-byte loads: block b reads the b-th of `blocks` contiguous ranges, its
// threads keeping kLoads consecutive 1 KiB-per-wave loads in flight, and writes one
// float per block to `sink` (so the loads are not elided; `sink` holds `blocks`
// floats). `blocks` = 0 picks 1024.
//
// saga_probe_stream_read_ex is the same read with `loads` (4, 8, 16 or 32) loads in
// flight per thread, and optionally a timeline: when `times` is not null it receives
// three values per block from the chip's constant-rate clock (s_memrealtime, 100 MHz):
// the block's first instruction, the arrival of its first load round's first load,
// and the block's last instruction (`times` holds 3 * blocks uint64 values).
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace {

constexpr int kThreads = 256;

template <int LOADS>
__global__ __launch_bounds__(kThreads) void k_stream_read(const uint4* __restrict__ p, size_t n16, size_t per_block,
                                                          float* sink, unsigned long long* times) {
  unsigned long long t0 = 0, t1 = 0;
  if (times) t0 = __builtin_amdgcn_s_memrealtime();
  const size_t base = (size_t)blockIdx.x * per_block;
  const size_t end = base + per_block < n16 ? base + per_block : n16;
  uint32_t acc = 0;
  bool first = true;
  for (size_t i = base + threadIdx.x; i < end; i += LOADS * kThreads) {
    uint4 v[LOADS];
#pragma unroll
    for (int u = 0; u < LOADS; ++u) {
      const size_t at = i + (size_t)u * kThreads;
      v[u] = at < end ? p[at] : make_uint4(0, 0, 0, 0);
    }
    if (first && times) {
      // loads complete in order: once at most LOADS - 1 are outstanding, the round's
      // first load has arrived
      __builtin_amdgcn_sched_barrier(0);
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(LOADS - 1) : "memory");
      t1 = __builtin_amdgcn_s_memrealtime();
      __builtin_amdgcn_sched_barrier(0);
    }
    first = false;
#pragma unroll
    for (int u = 0; u < LOADS; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  __shared__ uint32_t s[kThreads];
  s[threadIdx.x] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = 0;
    for (int t = 0; t < kThreads; ++t) r ^= s[t];
    sink[blockIdx.x] = __uint_as_float(r & 0x007fffffu);  // a finite value
    if (times) {
      const unsigned long long t2 = __builtin_amdgcn_s_memrealtime();
      times[3 * (size_t)blockIdx.x] = t0;
      times[3 * (size_t)blockIdx.x + 1] = t1;
      times[3 * (size_t)blockIdx.x + 2] = t2;
    }
  }
}

template <int LOADS>
int launch(const void* p, size_t bytes, float* sink, int blocks, unsigned long long* times, void* stream) {
  const size_t n16 = bytes / 16;
  const size_t per_block = (n16 + blocks - 1) / blocks;
  (void)hipGetLastError();
  hipLaunchKernelGGL(k_stream_read<LOADS>, dim3(blocks), dim3(kThreads), 0, (hipStream_t)stream,
                     reinterpret_cast<const uint4*>(p), n16, per_block, sink, times);
  return hipGetLastError() == hipSuccess ? 0 : 5;
}

}  // namespace

extern "C" int saga_probe_stream_read_ex(const void* p, size_t bytes, float* sink, int blocks, int loads,
                                         unsigned long long* times, void* stream) {
  if (!p || !sink || bytes % 16 != 0 || blocks < 1 || blocks > 65535) return 1;
  switch (loads) {
    case 4: return launch<4>(p, bytes, sink, blocks, times, stream);
    case 8: return launch<8>(p, bytes, sink, blocks, times, stream);
    case 16: return launch<16>(p, bytes, sink, blocks, times, stream);
    case 32: return launch<32>(p, bytes, sink, blocks, times, stream);
    default: return 1;
  }
}

extern "C" int saga_probe_stream_read(const void* p, size_t bytes, float* sink, int blocks, void* stream) {
  if (blocks < 0) return 1;
  return saga_probe_stream_read_ex(p, bytes, sink, blocks == 0 ? 1024 : blocks, 8, nullptr, stream);
}
