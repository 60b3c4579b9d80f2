// Time-parallel form of the sparse gated-delta scan, for gfx950.
//
// The scan ("Sparse Delta Memory", gist.science summaries of paper 2607.07386;
// Spanish page "Mecanismo Central" items 3 and 4) touches only the selected
// rows, and rows never interact: row s of stream (b,h) sees exactly the write
// and read events that name s, in time order.  So instead of walking time
// token by token, this path walks slots:
//   1. every event becomes a key (stream, slot, t, kind) with kind 0 for a write
//      and 1 for a read, so a token's write of a slot sorts before its read of
//      it (reads see the row after the write), and a payload (token, rank);
//   2. one radix sort (rocPRIM) over the bits the keys use orders all events of
//      a stream by slot, then time;
//   3. one lane group per slot segment loads the row once, applies its writes
//      in time order with the same roundings as the sequential scan, and stores
//      the row it holds at each read into a read buffer [S][T][R][d_v];
//   4. each token's output is the rank-ordered weighted sum of its read rows.
// The table and the outputs are bit-identical to the sequential scan's
// oracle (the same fp32 operations in the same order per element).  The work
// is independent of how many streams there are: the parallelism is the number
// of touched slots.
#include <hip/hip_runtime.h>
#include <rocprim/device/device_radix_sort.hpp>
#include <stdint.h>

#include "scan_common.h"
#include "sdm_internal.h"

namespace sdm {

using namespace scanc;

namespace {

constexpr int kSegChunk = 128;  // events per lane group's chunk

__device__ __forceinline__ int bits_for(int64_t n) {  // bits to hold 0 .. n-1
  int b = 0;
  while ((int64_t{1} << b) < n) b++;
  return b;
}

// 1. keys and payloads, one thread per event.  Payload: the event's position
// t*(W+R) + j in the stream (j < W: write rank j, else read rank j - W).
__global__ void __launch_bounds__(256) sdm_tp_keys_kernel(TpArgs a, uint64_t* keys,
                                                          uint32_t* vals) {
  const int WR = a.W + a.R;
  const int64_t n = (int64_t)a.S * a.T * WR;
  const int nb = bits_for(a.N), tb = bits_for(a.T);
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n;
       e += (int64_t)gridDim.x * blockDim.x) {
    const int64_t tok = e / WR;  // st * T + t
    const int j = (int)(e - tok * WR);
    const int64_t st = tok / a.T;
    const int t = (int)(tok - st * a.T);
    const bool rd = j >= a.W;
    const int32_t slot = rd ? a.ridx[tok * a.R + (j - a.W)] : a.widx[tok * a.W + j];
    keys[e] = ((((uint64_t)st << nb) | (uint64_t)(uint32_t)slot) << (tb + 1)) |
              ((uint64_t)t << 1) | (rd ? 1u : 0u);
    vals[e] = (uint32_t)(t * WR + j);
  }
}

// 3. slot segments.  A lane group takes the segments that start in its chunk
// of the sorted events (following each to its end, past the chunk if need be).
template <int LPR, bool VBF16>
__global__ void __launch_bounds__(256) sdm_tp_segments_kernel(TpArgs a, const uint64_t* keys,
                                                              const uint32_t* vals,
                                                              float* readbuf) {
#pragma clang fp contract(off)
  const int lane = threadIdx.x & 63;
  const int l = lane % LPR;
  const int64_t grp = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) / LPR;
  const int64_t n = (int64_t)a.S * a.T * (a.W + a.R);
  int64_t i = grp * kSegChunk;
  if (i >= n) return;  // no cross-lane operation follows
  const int64_t end = min(n, i + kSegChunk);
  const int nb = bits_for(a.N), tb = bits_for(a.T);
  const int WR = a.W + a.R;
  const int c0 = 4 * l;
  auto seg = [&](uint64_t k) { return k >> (tb + 1); };  // (stream, slot)
  if (i > 0) {
    const uint64_t prev = seg(keys[i - 1]);
    while (i < end && seg(keys[i]) == prev) i++;
  }
  if (i >= end) return;
  // keys and payloads two events ahead: the next segment's row and this
  // event's gates and v are in flight together
  auto rowp = [&](uint64_t sg) {
    const int64_t st = (int64_t)(sg >> nb);
    const int64_t slot = (int64_t)(sg & ((uint64_t{1} << nb) - 1));
    return a.M + (st * a.N + slot) * a.d_v + c0;
  };
  uint64_t scur = seg(keys[i]);
  uint32_t pj = vals[i];
  bool more1 = i + 1 < n;
  uint64_t k1 = more1 ? keys[i + 1] : ~uint64_t{0};
  uint32_t p1 = more1 ? vals[i + 1] : 0u;
  float* row = rowp(scur);
  float4 m = *reinterpret_cast<const float4*>(row);
  for (int64_t j = i;; j++) {
    const bool more2 = j + 2 < n;
    const uint64_t k2 = more2 ? keys[j + 2] : ~uint64_t{0};
    const uint32_t p2 = more2 ? vals[j + 2] : 0u;
    const uint64_t s1 = seg(k1);
    const bool ends = !more1 || s1 != scur;         // event j closes its segment
    const bool next_here = more1 && ends && j + 1 < end;  // and the next one is ours
    float* row1 = next_here ? rowp(s1) : row;
    const float4 mnext = *reinterpret_cast<const float4*>(row1);  // (row itself if unused)
    const int64_t st = (int64_t)(scur >> nb);
    const int t = (int)(pj / WR), r = (int)(pj - (uint32_t)t * WR);
    const int64_t tok = st * a.T + t;
    if (r < a.W) {
      const float c = a.beta[tok] * a.wwt[tok * a.W + r];
      const float omc = 1.0f - c;
      const float al = a.alpha[tok];
      const float4 v = load_v4(a.v, VBF16, tok * a.d_v + c0);
      m.x = omc * (al * m.x) + c * v.x;
      m.y = omc * (al * m.y) + c * v.y;
      m.z = omc * (al * m.z) + c * v.z;
      m.w = omc * (al * m.w) + c * v.w;
    } else {
      *reinterpret_cast<float4*>(readbuf + (tok * a.R + (r - a.W)) * a.d_v + c0) = m;
    }
    if (ends) {
      *reinterpret_cast<float4*>(row) = m;
      if (!next_here) break;  // no more events, or the next segment is the next chunk's
      scur = s1;
      row = row1;
      m = mnext;
    }
    pj = p1;
    more1 = more2;
    k1 = k2;
    p1 = p2;
  }
}

// 4. out[tok] = sum over r ascending of rwt[tok][r] * readbuf[tok][r], one
// thread per (token, 4 columns); separate multiply and add, as the oracle.
__global__ void __launch_bounds__(256) sdm_tp_reduce_kernel(TpArgs a, const float* readbuf) {
#pragma clang fp contract(off)
  const int q = a.d_v / 4;
  const int64_t n = (int64_t)a.S * a.T * q;
  for (int64_t x = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; x < n;
       x += (int64_t)gridDim.x * blockDim.x) {
    const int64_t tok = x / q;
    const int c0 = 4 * (int)(x - tok * q);
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int r = 0; r < a.R; r++) {
      const float w = a.rwt[tok * a.R + r];
      const float4 v = *reinterpret_cast<const float4*>(readbuf + (tok * a.R + r) * a.d_v + c0);
      acc.x = acc.x + w * v.x;
      acc.y = acc.y + w * v.y;
      acc.z = acc.z + w * v.z;
      acc.w = acc.w + w * v.w;
    }
    *reinterpret_cast<float4*>(a.out + tok * a.d_v + c0) = acc;
  }
}

size_t align256(size_t x) { return (x + 255) & ~size_t{255}; }

int host_bits(int64_t n) {
  int b = 0;
  while ((int64_t{1} << b) < n) b++;
  return b;
}

// rocPRIM's scratch for n pairs (a query; nothing runs)
size_t sort_temp_bytes(int64_t n, int end_bit) {
  size_t bytes = 0;
  const hipError_t e =
      rocprim::radix_sort_pairs(nullptr, bytes, (const uint64_t*)nullptr, (uint64_t*)nullptr,
                                (const uint32_t*)nullptr, (uint32_t*)nullptr, (size_t)n, 0,
                                (unsigned)end_bit);
  return e == hipSuccess ? bytes : SIZE_MAX / 4;  // an unmet size rather than a wrong one
}

}  // namespace

int tp_key_bits(int S, int T, int64_t N) { return host_bits(S) + host_bits(N) + host_bits(T) + 1; }

size_t tp_workspace_bytes(int S, int T, int64_t N, int d_v, int W, int R) {
  const int64_t n = (int64_t)S * T * (W + R);
  const int end_bit = tp_key_bits(S, T, N);
  return 2 * align256(n * 8) + 2 * align256(n * 4) + align256(sort_temp_bytes(n, end_bit)) +
         align256((size_t)S * T * R * d_v * 4);
}

hipError_t launch_scan_tp(const TpArgs& a, bool vbf16, void* ws, hipStream_t stream) {
  const int64_t n = (int64_t)a.S * a.T * (a.W + a.R);
  if (n == 0) return hipSuccess;
  const int end_bit = tp_key_bits(a.S, a.T, a.N);
  unsigned char* p = static_cast<unsigned char*>(ws);
  uint64_t* k_in = reinterpret_cast<uint64_t*>(p);
  p += align256(n * 8);
  uint64_t* k_out = reinterpret_cast<uint64_t*>(p);
  p += align256(n * 8);
  uint32_t* v_in = reinterpret_cast<uint32_t*>(p);
  p += align256(n * 4);
  uint32_t* v_out = reinterpret_cast<uint32_t*>(p);
  p += align256(n * 4);
  size_t tmp_bytes = sort_temp_bytes(n, end_bit);
  void* tmp = p;
  p += align256(tmp_bytes);
  float* readbuf = reinterpret_cast<float*>(p);

  int grid = (int)std::min<int64_t>((n + 255) / 256, 65536);
  hipLaunchKernelGGL(sdm_tp_keys_kernel, dim3(grid), dim3(256), 0, stream, a, k_in, v_in);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = rocprim::radix_sort_pairs(tmp, tmp_bytes, k_in, k_out, v_in, v_out, (size_t)n, 0,
                                (unsigned)end_bit, stream);
  if (e != hipSuccess) return e;
  const int lpr = a.d_v / 4;
  const int64_t groups = (n + kSegChunk - 1) / kSegChunk;
  const int64_t threads = groups * lpr;
  const unsigned sgrid = (unsigned)((threads + 255) / 256);
#define SDM_TP_SEG(LPR_)                                                                      \
  if (lpr == LPR_) {                                                                          \
    if (vbf16)                                                                                \
      hipLaunchKernelGGL((sdm_tp_segments_kernel<LPR_, true>), dim3(sgrid), dim3(256), 0,     \
                         stream, a, k_out, v_out, readbuf);                                   \
    else                                                                                      \
      hipLaunchKernelGGL((sdm_tp_segments_kernel<LPR_, false>), dim3(sgrid), dim3(256), 0,    \
                         stream, a, k_out, v_out, readbuf);                                   \
  } else
  SDM_TP_SEG(4) SDM_TP_SEG(8) SDM_TP_SEG(16) SDM_TP_SEG(32) SDM_TP_SEG(64) {
    return hipErrorInvalidValue;
  }
#undef SDM_TP_SEG
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t nr = (int64_t)a.S * a.T * (a.d_v / 4);
  const int rgrid = (int)std::min<int64_t>((nr + 255) / 256, 65536);
  hipLaunchKernelGGL(sdm_tp_reduce_kernel, dim3(rgrid), dim3(256), 0, stream, a, readbuf);
  return hipGetLastError();
}

}  // namespace sdm
