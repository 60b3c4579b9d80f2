// Routed slots with selective decay (Raven-style writes on the memory table),
// for gfx950: the router.
//
// Spanish page "Resumen Tecnico: Raven", section 2.2: per token, sigmoid
// scores m = sigmoid(z) over the M slots, only the K largest kept and
// normalised (r = m / sum of the kept m), and the routed slots decay toward the
// token's content with gamma = exp(a_t * r), every other slot frozen.  The
// write S[i] = gamma*S[i] + (1-gamma)*u is the scan's write with alpha = beta = 1
// and weight c = 1 - gamma, so the router emits c and the table update runs in
// sdm_scan.  Selection is on the logits (sigmoid is strictly increasing), with
// ties to the lower slot index.
//
// One wave per (token, side).  The logits become order-preserving 32-bit keys
// in LDS; a 4-digit radix select (8-bit digits, LDS histogram, suffix counts by
// lane shuffles) finds the K-th largest key and how many keys equal to it are
// taken (lowest indices first); the K winners are ranked by (key desc, index
// asc) with one comparison sweep over the winner list, and written in rank
// order with their gates.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "sdm_internal.h"

namespace sdm {

namespace {

constexpr int kRouteWaves = 4;

__device__ __forceinline__ uint32_t okey(float z) {
  const uint32_t u = __float_as_uint(z + 0.0f);  // -0 -> +0
  return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}

__global__ void __launch_bounds__(kRouteWaves * 64) sdm_route_kernel(RouteArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int M = a.M, K = a.K;
  uint32_t* keys = reinterpret_cast<uint32_t*>(smem) + (size_t)wave * (M + 256 + 2 * K);
  uint32_t* hist = keys + M;
  uint32_t* wkey = hist + 256;  // winners: key, then index
  int32_t* widxl = reinterpret_cast<int32_t*>(wkey + K);

  const int64_t unit = (int64_t)blockIdx.x * (kRouteWaves / 2) + (wave >> 1);
  const int side = wave & 1;
  if (unit >= a.units) return;  // wave-uniform; no barrier below
  const float* z = (side ? a.zq : a.zk) + unit * M;
  const uint64_t below = (1ull << lane) - 1ull;

  for (int i = lane; i < M; i += 64) keys[i] = okey(z[i]);

  // ---- radix select of the K-th largest key ------------------------------
  uint32_t prefix = 0, pmask = 0;
  int need = K;  // keys still to take at or below the current prefix
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = lane; i < 256; i += 64) hist[i] = 0;
    wave_lds_sync();
    for (int i = lane; i < M; i += 64) {
      const uint32_t k = keys[i];
      if ((k & pmask) == prefix) atomicAdd(&hist[(k >> shift) & 255], 1u);
    }
    wave_lds_sync();
    // lane l holds bins 4l..4l+3; suffix counts from the top bin down
    uint32_t c[4];
#pragma unroll
    for (int j = 0; j < 4; j++) c[j] = hist[4 * lane + j];
    const uint32_t mine = c[0] + c[1] + c[2] + c[3];
    // inclusive suffix scan over lanes (lane 63 holds the top bins)
    uint32_t suf = mine;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t x = __shfl_down(suf, o);
      if (lane + o < 64) suf += x;
    }
    const uint32_t above = suf - mine;  // keys in bins of higher lanes
    // the digit: the bin where the count from the top first reaches `need`
    int found = -1;
    uint32_t before = 0;
    uint32_t run = above;
#pragma unroll
    for (int j = 3; j >= 0; j--) {
      if (found < 0 && run < (uint32_t)need && run + c[j] >= (uint32_t)need) {
        found = 4 * lane + j;
        before = run;
      }
      run += c[j];
    }
    const uint64_t hit = __ballot(found >= 0);
    const int src = __builtin_ctzll(hit);
    const int digit = __shfl(found, src);
    need -= (int)__shfl(before, src);
    prefix |= (uint32_t)digit << shift;
    pmask |= 255u << shift;
    wave_lds_sync();
  }
  const uint32_t kth = prefix;  // the K-th largest key; `need` of its copies are taken

  // ---- winners in index order ---------------------------------------------
  int nsel = 0, eq = 0;
  for (int base = 0; base < M; base += 64) {
    const int i = base + lane;
    const uint32_t k = i < M ? keys[i] : 0u;
    const bool isq = i < M && k == kth;
    const uint64_t beq = __ballot(isq);
    const bool take = i < M && (k > kth || (isq && eq + __popcll(beq & below) < need));
    const uint64_t bt = __ballot(take);
    if (take) {
      const int pos = nsel + __popcll(bt & below);
      wkey[pos] = k;
      widxl[pos] = i;
    }
    nsel += __popcll(bt);
    eq += __popcll(beq);
  }
  wave_lds_sync();

  // ---- rank, gates, output --------------------------------------------------
  int rank[2], sidx[2];
  float m[2];
  float msum = 0.f;
#pragma unroll
  for (int u = 0; u < 2; u++) {
    const int p = u * 64 + lane;
    rank[u] = 0;
    sidx[u] = 0;
    m[u] = 0.f;
    if (p < K) {
      const uint32_t k = wkey[p];
      const int ix = min(max(widxl[p], 0), M - 1);  // the list holds exactly K winners
      int r = 0;
      for (int q = 0; q < K; q++) {
        const uint32_t kq = wkey[q];
        r += (kq > k || (kq == k && widxl[q] < ix)) ? 1 : 0;
      }
      rank[u] = r;
      sidx[u] = ix;
      m[u] = 1.0f / (1.0f + expf(-z[ix]));
      msum += m[u];
    }
  }
  for (int o = 32; o > 0; o >>= 1) msum += __shfl_xor(msum, o);
  const float al = side ? 0.f : a.a[unit];
  int32_t* oidx = (side ? a.ridx : a.widx) + unit * K;
  float* oval = (side ? a.rwt : a.wcoef) + unit * K;
#pragma unroll
  for (int u = 0; u < 2; u++) {
    if (u * 64 + lane < K) {
      const float r = m[u] / msum;
      oidx[rank[u]] = sidx[u];
      oval[rank[u]] = side ? r : -expm1f(al * r);
    }
  }
}

}  // namespace

size_t route_lds_bytes(int M, int K) {
  return (size_t)kRouteWaves * (M + 256 + 2 * K) * sizeof(uint32_t);
}

hipError_t launch_route(const RouteArgs& a, hipStream_t stream) {
  if (a.units == 0) return hipSuccess;
  const int64_t grid = (a.units + kRouteWaves / 2 - 1) / (kRouteWaves / 2);
  const size_t lds = route_lds_bytes(a.M, a.K);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(sdm_route_kernel),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(sdm_route_kernel, dim3((unsigned)grid), dim3(kRouteWaves * 64), lds, stream,
                     a);
  return hipGetLastError();
}

}  // namespace sdm
