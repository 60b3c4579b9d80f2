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
// One wave per (token, side), in one of two forms.
//   * M <= 1024 slots: each lane holds the keys of slots lane, lane + 64, ...
//     in registers as unique 64-bit keys (order-preserving logit bits, then the
//     complemented slot).  A first threshold at the Gaussian quantile of the
//     logits' mean and spread, then bisection on keys, leaves between K and
//     cap_for(K) candidates.  They are compacted to LDS and sorted by a
//     register bitonic network, and the first K are written in rank order with
//     their gates.  The selection helpers are the addressing kernel's.
//   * Larger M: the logits become order-preserving 32-bit keys in LDS.  A
//     4-digit radix select (8-bit digits, LDS histogram, suffix counts by lane
//     shuffles) finds the K-th largest key and how many keys equal to it are
//     taken (lowest indices first).  The K winners are ranked by (key desc,
//     index asc) with one comparison sweep over the winner list, and written
//     in rank order with their gates.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "score_topk_impl.h"
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

// The K best of c sorted candidates in buf (descending keys), as slots and
// gates in rank order: m = sigmoid(logit), r = m / (sum of the K kept m).
template <int E>
__device__ __forceinline__ void route_emit(const uint64_t* buf, int c, int K, int lane, int side,
                                           float al, int32_t* oidx, float* oval) {
  uint64_t v[E];
#pragma unroll
  for (int r = 0; r < E; r++) {
    const int i = lane * E + r;
    v[r] = i < c ? buf[i] : 0ull;
  }
  bitonic_desc<E>(v, lane);
  float m[E];
  float msum = 0.f;
#pragma unroll
  for (int r = 0; r < E; r++) {
    const int p = lane * E + r;
    m[r] = p < K ? 1.0f / (1.0f + expf(-key_score(v[r]))) : 0.f;
    msum += m[r];
  }
  msum = wave_sum(msum);
#pragma unroll
  for (int r = 0; r < E; r++) {
    const int p = lane * E + r;
    if (p < K) {
      const float rr = m[r] / msum;
      oidx[p] = (int32_t)key_id(v[r]);
      oval[p] = side ? rr : -expm1f(al * rr);
    }
  }
}

// Register form for M <= 64*KPL slots; zg: Gaussian quantile of the first
// threshold (about 1.4K of the M logits above mean + zg * spread).
template <int KPL>
__global__ void __launch_bounds__(kRouteWaves * 64) sdm_route_reg_kernel(RouteArgs a, float zg) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int M = a.M, K = a.K;
  uint64_t* buf = reinterpret_cast<uint64_t*>(smem) + (size_t)wave * kCapMax;
  const int64_t unit = (int64_t)blockIdx.x * (kRouteWaves / 2) + (wave >> 1);
  const int side = wave & 1;
  if (unit >= a.units) return;  // wave-uniform; no barrier below
  const float* z = (side ? a.zq : a.zk) + unit * M;

  uint64_t key[KPL];
  float sum = 0.f, sq = 0.f;
  uint32_t mo = 0u;  // largest logit code
#pragma unroll
  for (int c = 0; c < KPL; c++) {
    const int i = c * 64 + lane;
    key[c] = 0ull;  // below every slot's key (whose low half is >= 1)
    if (i < M) {
      const float v = z[i];
      key[c] = make_key(v, (uint32_t)i);
      mo = max(mo, (uint32_t)(key[c] >> 32));
      sum += v;
      sq += v * v;
    }
  }
  mo = wave_max32(mo);
  sum = wave_sum(sum);
  sq = wave_sum(sq);
  const float mean = sum / M;
  const float sd = sqrtf(fmaxf(sq / M - mean * mean, 0.f));
  const uint64_t guess = (uint64_t)ord32(mean + zg * sd) << 32;
  // K <= M slot keys are >= 1, so the threshold never admits the padding and
  // leaves between K and cap_for(K) <= kCapMax keys
  const uint64_t t =
      find_threshold<KPL>(key, K, cap_for(K), guess, 0ull, ((uint64_t)mo + 1ull) << 32);
  const int c = compact_ge<KPL>(key, t, buf, lane);
  wave_lds_sync();
  const float al = side ? 0.f : a.a[unit];
  int32_t* oidx = (side ? a.ridx : a.widx) + unit * K;
  float* oval = (side ? a.rwt : a.wcoef) + unit * K;
  if (c <= 64) route_emit<1>(buf, c, K, lane, side, al, oidx, oval);
  else if (c <= 128) route_emit<2>(buf, c, K, lane, side, al, oidx, oval);
  else route_emit<4>(buf, c, K, lane, side, al, oidx, oval);
}

constexpr int kRouteRegMax = 1024;  // largest M of the register form

}  // namespace

size_t route_lds_bytes(int M, int K) {
  if (M <= kRouteRegMax) return (size_t)kRouteWaves * kCapMax * sizeof(uint64_t);
  return (size_t)kRouteWaves * (M + 256 + 2 * K) * sizeof(uint32_t);
}

hipError_t launch_route(const RouteArgs& a, hipStream_t stream) {
  if (a.units == 0) return hipSuccess;
  const int64_t grid = (a.units + kRouteWaves / 2 - 1) / (kRouteWaves / 2);
  const size_t lds = route_lds_bytes(a.M, a.K);
  if (a.M <= kRouteRegMax) {
    const float zg = guess_z(a.K, a.M);
    auto launch = [&](auto kern) {
      hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kRouteWaves * 64), lds, stream, a, zg);
      return hipGetLastError();
    };
    if (a.M <= 64) return launch(sdm_route_reg_kernel<1>);
    if (a.M <= 128) return launch(sdm_route_reg_kernel<2>);
    if (a.M <= 256) return launch(sdm_route_reg_kernel<4>);
    if (a.M <= 512) return launch(sdm_route_reg_kernel<8>);
    return launch(sdm_route_reg_kernel<16>);
  }
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(sdm_route_kernel),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(sdm_route_kernel, dim3((unsigned)grid), dim3(kRouteWaves * 64), lds, stream,
                     a);
  return hipGetLastError();
}

}  // namespace sdm
