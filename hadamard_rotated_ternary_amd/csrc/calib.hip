// Plain streaming read (measurement helper; declared in hbl_calib.h).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hbl_calib.h"

namespace {

constexpr int kThreads = 512;
constexpr int kUnitsPerThread = 8;
constexpr size_t kChunkUnits = (size_t)kThreads * kUnitsPerThread;   // 4096 units of 16 bytes = 64 KiB

// Workgroup b reads units [b * 4096, (b + 1) * 4096) clipped to n: load i of
// thread t is unit b * 4096 + 512 i + t, so each wave instruction covers 64
// consecutive units (1 KiB).  All eight loads are issued before the first is
// used; the XOR keeps them from being removed.  n >= 1 (checked by the caller).
__global__ __launch_bounds__(kThreads) void stream_read_kernel(const uint4* __restrict__ src, size_t n,
                                                                uint32_t* __restrict__ digest) {
  const size_t base = (size_t)blockIdx.x * kChunkUnits + threadIdx.x;
  // loads are unconditional (indices past n clamped to the last unit, their
  // values dropped below), so none waits behind a branch
  uint4 v[kUnitsPerThread];
#pragma unroll
  for (int i = 0; i < kUnitsPerThread; ++i) {
    const size_t u = base + (size_t)i * kThreads;
    v[i] = src[u < n ? u : n - 1];
  }
  uint32_t x = 0;
#pragma unroll
  for (int i = 0; i < kUnitsPerThread; ++i)
    if (base + (size_t)i * kThreads < n) x ^= v[i].x ^ v[i].y ^ v[i].z ^ v[i].w;
  // wave XOR, then across the eight waves through LDS
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x ^= (uint32_t)__shfl_xor((int)x, o, 64);
  __shared__ uint32_t part[kThreads / 64];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t s = 0;
#pragma unroll
    for (int w = 0; w < kThreads / 64; ++w) s ^= part[w];
    digest[blockIdx.x] = s;
  }
}

// Every workgroup reads units [0, n): pass j of thread t loads units
// 4096 j + 512 i + t (i < 8, clamped to n - 1 and dropped past it).
__global__ __launch_bounds__(kThreads) void broadcast_read_kernel(const uint4* __restrict__ src, size_t n,
                                                                   uint32_t* __restrict__ digest) {
  uint32_t x = 0;
  for (size_t b0 = 0; b0 < n; b0 += kChunkUnits) {
    const size_t base = b0 + threadIdx.x;
    uint4 v[kUnitsPerThread];
#pragma unroll
    for (int i = 0; i < kUnitsPerThread; ++i) {
      const size_t u = base + (size_t)i * kThreads;
      v[i] = src[u < n ? u : n - 1];
    }
#pragma unroll
    for (int i = 0; i < kUnitsPerThread; ++i)
      if (base + (size_t)i * kThreads < n) x ^= v[i].x ^ v[i].y ^ v[i].z ^ v[i].w;
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x ^= (uint32_t)__shfl_xor((int)x, o, 64);
  __shared__ uint32_t part[kThreads / 64];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t s = 0;
#pragma unroll
    for (int w = 0; w < kThreads / 64; ++w) s ^= part[w];
    digest[blockIdx.x] = s;
  }
}

}  // namespace

extern "C" int hbl_calib_broadcast_read(const void* src, size_t bytes, unsigned workgroups, uint32_t* digest,
                                        hipStream_t stream) {
  if (src == nullptr || digest == nullptr) return 1;
  if (bytes == 0 || bytes % 16 != 0 || workgroups == 0 || workgroups > 65536) return 2;
  if (reinterpret_cast<uintptr_t>(src) % 16 != 0 || reinterpret_cast<uintptr_t>(digest) % 4 != 0) return 4;
  hipLaunchKernelGGL(broadcast_read_kernel, dim3(workgroups), dim3(kThreads), 0, stream,
                     static_cast<const uint4*>(src), bytes / 16, digest);
  return hipGetLastError() == hipSuccess ? 0 : 6;
}

extern "C" int hbl_calib_stream_read(const void* src, size_t bytes, uint32_t* digest, hipStream_t stream) {
  if (src == nullptr || digest == nullptr) return 1;
  if (bytes == 0 || bytes % 16 != 0) return 2;
  if (reinterpret_cast<uintptr_t>(src) % 16 != 0 || reinterpret_cast<uintptr_t>(digest) % 4 != 0) return 4;
  const size_t n = bytes / 16;
  const size_t grid = (n + kChunkUnits - 1) / kChunkUnits;
  if (grid > 0x7fffffffu) return 2;
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)grid), dim3(kThreads), 0, stream,
                     static_cast<const uint4*>(src), n, digest);
  return hipGetLastError() == hipSuccess ? 0 : 6;
}
