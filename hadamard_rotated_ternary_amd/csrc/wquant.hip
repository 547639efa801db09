// Offline per-tensor absmean ternarisation of latent weights and 2-bit packing.
//
// QbitAI article on BitNet v2, section 引入H-BitLinear模块, and 新智元 article
// "微软再放LLM量化大招", section H-BitLinear模块: weights are mapped to
// {-1, 0, 1} with a single per-tensor scale, the mean of |W|.
//
// The sum of |W| is taken in fp64 in a fixed order (64-column blocks of each
// row, the block sums in order, then the row sums in row order), so alpha is
// reproducible from call to call; any fp64 order is far more precise than the
// fp32 result, which stays within one ulp of the exactly rounded mean.
// Code(w) = round-half-even(w / a) clamped to [-1, 1] is nonzero exactly when
// |w| > a / 2 (a tie rounds to 0), and 0.5f * a is exact in fp32, so the
// kernel decides with one comparison instead of a division.
#include "common.h"
#include "launch.h"

namespace hbl {

// Row sums of |w| in fp64 in a fixed order: 64-column blocks, each summed
// left to right, block sums added left to right.  One 256-thread workgroup
// per row: the row is staged through LDS 16384 columns at a time with
// coalesced 16-byte loads (blocks padded to 65 floats so the per-block walks
// hit distinct banks), thread b sums block b of the chunk, and thread 0 adds
// all block sums (at most 512, K <= 32768) in order.
__global__ __launch_bounds__(256) void wrowsum_kernel(const float* __restrict__ w, int N, int K,
                                                     double* __restrict__ rowsum) {
  constexpr int CHUNK = 16384;
  __shared__ float row[256 * 65];
  __shared__ double bsum[512];
  const int n = blockIdx.x, t = threadIdx.x;
  for (int c0 = 0; c0 < K; c0 += CHUNK) {
    const int len = K - c0 < CHUNK ? K - c0 : CHUNK;
    const float4* src = reinterpret_cast<const float4*>(w + (size_t)n * K + c0);
    for (int i = t; i < len / 4; i += 256) {
      const float4 v = src[i];
      const int e = 4 * i, b = e >> 6, o = e & 63;
      float* d = row + b * 65 + o;
      d[0] = v.x; d[1] = v.y; d[2] = v.z; d[3] = v.w;
    }
    __syncthreads();
    if (t < (len + 63) / 64) {
      const int bl = len - 64 * t < 64 ? len - 64 * t : 64;
      double acc = 0.0;
      for (int o = 0; o < bl; ++o) acc += (double)fabsf(row[t * 65 + o]);
      bsum[c0 / 64 + t] = acc;
    }
    __syncthreads();   // the row buffer is refilled by the next chunk
  }
  if (t == 0) {
    const int nb = (K + 63) / 64;
    double acc = 0.0;
    for (int b = 0; b < nb; ++b) acc += bsum[b];
    rowsum[n] = acc;
  }
}

// alpha = fp32(sum_n rowsum[n] / (N K)), summed in row order by one thread;
// the row sums are staged through LDS 2048 at a time (coalesced loads) so the
// ordered sum does not wait on one global load per row.
__global__ __launch_bounds__(256) void walpha_kernel(const double* __restrict__ rowsum, int N, int K,
                                                    float* __restrict__ walpha) {
  __shared__ double chunk[2048];
  double s = 0.0;
  for (int n0 = 0; n0 < N; n0 += 2048) {
    const int cnt = N - n0 < 2048 ? N - n0 : 2048;
    for (int i = threadIdx.x; i < cnt; i += 256) chunk[i] = rowsum[n0 + i];
    __syncthreads();
    if (threadIdx.x == 0)
      for (int i = 0; i < cnt; ++i) s += chunk[i];
    __syncthreads();
  }
  if (threadIdx.x == 0) walpha[0] = (float)(s / ((double)N * (double)K));
}

// One thread per packed 32-bit word (16 consecutive k of one row), stored at
// its tiled position (wword).
__global__ __launch_bounds__(256) void wpack_kernel(const float* __restrict__ w, int N, int K,
                                                   const float* __restrict__ walpha,
                                                   uint32_t* __restrict__ wpack) {
  const size_t words = (size_t)N * (K / 16);
  const size_t q = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (q >= words) return;
  const float a = fmaxf(walpha[0], kEpsQ);
  const float half = 0.5f * a;
  const float4* src = reinterpret_cast<const float4*>(w + q * 16);
  uint32_t word = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float4 f = src[j];
    const float e[4] = {f.x, f.y, f.z, f.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // element 4j+i of this group of 16: k0 + 4j + i -> bits 8i + 2j
      const float x = e[i];
      const uint32_t code = fabsf(x) > half ? (x > 0.f ? 1u : 3u) : 0u;
      word |= code << (8 * i + 2 * j);
    }
  }
  const int wpr = K / 16;
  wpack[wword((int)(q / wpr), (int)(q % wpr), K)] = word;
}

__global__ __launch_bounds__(256) void wunpack_kernel(const uint32_t* __restrict__ wpack, int N, int K,
                                                     int8_t* __restrict__ wt) {
  const size_t words = (size_t)N * (K / 16);
  const size_t q = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (q >= words) return;
  const int wpr = K / 16;
  const uint32_t p = wpack[wword((int)(q / wpr), (int)(q % wpr), K)];
  uint32_t out[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    out[j] = __builtin_amdgcn_perm(0u, 0xFF000100u, (p >> (2 * j)) & 0x03030303u);
  *reinterpret_cast<uint4*>(wt + q * 16) = make_uint4(out[0], out[1], out[2], out[3]);
}

hipError_t launch_wquant(const WquantArgs& a) {
  hipLaunchKernelGGL(wrowsum_kernel, dim3(a.N), dim3(256), 0, a.stream, a.w, a.N, a.K, a.rowsum);
  hipLaunchKernelGGL(walpha_kernel, dim3(1), dim3(256), 0, a.stream, a.rowsum, a.N, a.K, a.walpha);
  const size_t words = (size_t)a.N * (a.K / 16);
  hipLaunchKernelGGL(wpack_kernel, dim3((unsigned)((words + 255) / 256)), dim3(256), 0, a.stream, a.w, a.N,
                     a.K, a.walpha, reinterpret_cast<uint32_t*>(a.wpack));
  return hipGetLastError();
}

hipError_t launch_unpack(const uint8_t* wpack, int N, int K, int8_t* wt, hipStream_t stream) {
  const size_t words = (size_t)N * (K / 16);
  hipLaunchKernelGGL(wunpack_kernel, dim3((unsigned)((words + 255) / 256)), dim3(256), 0, stream,
                     reinterpret_cast<const uint32_t*>(wpack), N, K, wt);
  return hipGetLastError();
}

}  // namespace hbl
