// Exclusive prefix sum of int32 counts on the device, for the library's
// counting sorts: x[0..n) is replaced by its exclusive prefix sums and x[n]
// receives the total.  Three launches: per-block sums, one workgroup scanning
// the block sums, then each block's own scan plus its offset.  Counts and
// their sums must fit in int32.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sdm {
namespace exsum {
namespace {  // one copy of the kernels per translation unit

constexpr int kPer = 16;           // elements per thread
constexpr int kBlock = 256 * kPer;  // elements per workgroup

// exclusive prefix of v over the 256 threads of the workgroup
__device__ __forceinline__ int block_excl256(int v, int* tmp) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int inc = v;
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(inc, o);
    if (lane >= o) inc += y;
  }
  if (lane == 63) tmp[w] = inc;
  __syncthreads();
  int before = 0;
  for (int i = 0; i < w; i++) before += tmp[i];
  __syncthreads();
  return before + inc - v;
}

__global__ void __launch_bounds__(256) sums_kernel(const int32_t* __restrict__ x, int64_t n,
                                                   int32_t* __restrict__ bsum) {
  __shared__ int tmp[4];
  const int64_t base = (int64_t)blockIdx.x * kBlock + (int64_t)threadIdx.x * kPer;
  int s = 0;
  for (int i = 0; i < kPer; i++) s += base + i < n ? x[base + i] : 0;
  const int ex = block_excl256(s, tmp);
  if (threadIdx.x == 255) bsum[blockIdx.x] = ex + s;
}

__global__ void __launch_bounds__(256) top_kernel(int32_t* __restrict__ bsum, int nb,
                                                  int32_t* __restrict__ total) {
  __shared__ int tmp[4];
  const int per = (nb + 255) / 256;
  const int b0 = threadIdx.x * per;
  int s = 0;
  for (int i = 0; i < per; i++) s += b0 + i < nb ? bsum[b0 + i] : 0;
  int run = block_excl256(s, tmp);
  for (int i = 0; i < per; i++) {
    if (b0 + i < nb) {
      const int v = bsum[b0 + i];
      bsum[b0 + i] = run;
      run += v;
    }
  }
  if (threadIdx.x == 255) *total = run;
}

__global__ void __launch_bounds__(256) down_kernel(int32_t* __restrict__ x, int64_t n,
                                                   const int32_t* __restrict__ bsum) {
  __shared__ int tmp[4];
  const int64_t base = (int64_t)blockIdx.x * kBlock + (int64_t)threadIdx.x * kPer;
  int v[kPer];
  int s = 0;
  for (int i = 0; i < kPer; i++) {
    v[i] = base + i < n ? x[base + i] : 0;
    s += v[i];
  }
  int run = block_excl256(s, tmp) + bsum[blockIdx.x];
  for (int i = 0; i < kPer; i++) {
    if (base + i < n) x[base + i] = run;
    run += v[i];
  }
}

// block sums needed for n elements
inline int64_t blocks(int64_t n) { return (n + kBlock - 1) / kBlock; }

// x: n + 1 int32 (counts in, exclusive sums and the total out); bsum: blocks(n) int32
inline hipError_t run(int32_t* x, int64_t n, int32_t* bsum, hipStream_t stream) {
  const int64_t nb = blocks(n);
  if (nb == 0) {
    hipLaunchKernelGGL(top_kernel, dim3(1), dim3(256), 0, stream, bsum, 0, x + n);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(sums_kernel, dim3((unsigned)nb), dim3(256), 0, stream, x, n, bsum);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(top_kernel, dim3(1), dim3(256), 0, stream, bsum, (int)nb, x + n);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(down_kernel, dim3((unsigned)nb), dim3(256), 0, stream, x, n, bsum);
  return hipGetLastError();
}

}  // namespace
}  // namespace exsum
}  // namespace sdm
