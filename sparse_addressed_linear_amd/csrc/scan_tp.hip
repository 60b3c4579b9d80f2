// Time-parallel form of the sparse gated-delta scan, for gfx950.
//
// The scan ("Sparse Delta Memory", gist.science summaries of paper 2607.07386;
// Spanish page "Mecanismo Central" items 3 and 4) touches only the selected
// rows, and rows never interact: row s of stream (b,h) sees exactly the write
// and read events that name s, in time order.  So instead of walking time
// token by token, this path walks slots:
//   1. a stream's events, listed in time order (token t's W writes, then its
//      R reads, at position t*(W+R) + j), are sorted stably by slot within
//      the stream.  A token's write of a slot therefore precedes its read of
//      it (reads see the row after the write).  The sort is a least
//      significant digit radix sort of the slot, at most 10 bits per pass: a
//      per-tile digit count, one exclusive sum over (stream, digit, tile),
//      and a stable scatter that sorts each tile by digit in LDS (ranking a
//      row of 64 events at once) before writing it out;
//   2. one lane group per slot segment loads the row once, applies its writes
//      in time order with the same roundings as the sequential scan, stores
//      the row it holds at each read into a read buffer [S][T][R][d_v], and
//      writes the row back if any write changed it;
//   3. each token's output is the rank-ordered weighted sum of its read rows.
// The table and the outputs are bit-identical to the sequential scan's
// oracle (the same fp32 operations in the same order per element).  The work
// is independent of how many streams there are: the parallelism is the number
// of touched slots.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "excl_sum.h"
#include "scan_common.h"
#include "sdm_internal.h"

namespace sdm {

using namespace scanc;

namespace {

constexpr int kSegChunk = 128;  // events per lane group's chunk
constexpr int kMaxDigit = 10;   // slot bits per sort pass
constexpr int kMaxRad = 1 << kMaxDigit;
constexpr int kTile = 4096;     // events per sort tile

// One pass of the slot sort: digit (slot >> shift) & (rad - 1) over tiles of
// kTile events of a stream.
struct SortPass {
  int64_t L;    // events per stream, T*(W+R)
  int64_t tps;  // tiles per stream
  int shift, dbits;
};

// slot named by the event at position p of stream st, in time order
// (positions are below 2^31)
__device__ __forceinline__ uint32_t event_slot(const TpArgs& a, int64_t st, int64_t p) {
  const uint32_t WR = (uint32_t)(a.W + a.R);
  const uint32_t t = (uint32_t)p / WR;
  const int j = (int)((uint32_t)p - t * WR);
  const int64_t tok = st * a.T + t;
  return (uint32_t)(j < a.W ? a.widx[tok * a.W + j] : a.ridx[tok * a.R + (j - a.W)]);
}

// An event whose slot lies outside [0, N) is ignored: it sorts as slot 0 with
// kIgnored set in its payload, writes nothing and reads a zero row.
constexpr uint32_t kIgnored = 0x80000000u;

__device__ __forceinline__ void first_pass_event(const TpArgs& a, int64_t st, int64_t p,
                                                 uint32_t& key, uint32_t& val) {
  const uint32_t s = event_slot(a, st, p);
  const bool ok = s < (uint32_t)a.N;
  key = ok ? s : 0u;
  val = ok ? (uint32_t)p : ((uint32_t)p | kIgnored);
}

// 1a. digit counts of each tile: gh[(stream*rad + digit)*tps + tile].  One
// wave per tile with its own LDS counts; the first pass reads the slots from
// the index lists, later ones the previous pass's output.
template <bool FIRST>
__global__ void __launch_bounds__(256) sdm_tp_hist_kernel(TpArgs a, SortPass sp,
                                                          const uint32_t* __restrict__ kin,
                                                          int32_t* __restrict__ gh) {
  __shared__ int32_t hist_all[4][kMaxRad];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t g = (int64_t)blockIdx.x * 4 + wave;
  if (g >= (int64_t)a.S * sp.tps) return;  // the whole wave; no workgroup barrier follows
  int32_t* hist = hist_all[wave];
  const int rad = 1 << sp.dbits;
  const int64_t st = g / sp.tps, tile = g - st * sp.tps;
  for (int d = lane; d < rad; d += 64) hist[d] = 0;
  const int64_t t0 = tile * kTile, t1 = std::min<int64_t>(sp.L, t0 + kTile);
  constexpr int kU = 8;  // a batch of loads in flight before any count
  for (int64_t p0 = t0 + lane; p0 < t1; p0 += 64 * kU) {
    uint32_t k[kU];
#pragma unroll
    for (int u = 0; u < kU; u++) {
      const int64_t p = p0 + 64 * u;
      uint32_t kf = 0u, vf;
      if (FIRST && p < t1) first_pass_event(a, st, p, kf, vf);
      k[u] = p < t1 ? (FIRST ? kf : kin[st * sp.L + p]) : 0u;
    }
#pragma unroll
    for (int u = 0; u < kU; u++)
      if (p0 + 64 * u < t1) atomicAdd(&hist[(k[u] >> sp.shift) & (rad - 1)], 1);
  }
  for (int d = lane; d < rad; d += 64) gh[(st * rad + d) * sp.tps + tile] = hist[d];
}

// 1b. stable scatter, one workgroup per tile.  The tile's events are sorted
// by digit in LDS first and then written out in that order, so the lanes of
// a wave store runs of neighbouring places.  In LDS, wave w walks its quarter
// of the tile in rows of 64 events: the lanes holding the same digit find
// each other with one ballot per digit bit, an event's place is its digit's
// next local place (after the tile's smaller digits and the earlier waves'
// events of the digit) plus the number of earlier lanes of the row with that
// digit, and the row's last lane of each digit moves that place on.  The
// global place is the local one shifted by the digit's exclusive sum of
// counts over (stream, digit, tile).
template <bool FIRST>
__global__ void __launch_bounds__(256) sdm_tp_scatter_kernel(
    TpArgs a, SortPass sp, const uint32_t* __restrict__ kin, const uint32_t* __restrict__ vin,
    const int32_t* __restrict__ offs, uint32_t* __restrict__ kout, uint32_t* __restrict__ vout) {
  constexpr int kU = kTile / 256;  // rows per wave
  constexpr int kPer = kMaxRad / 256;  // digits per thread in the exclusive sum, at most
  __shared__ uint32_t sk[kTile], sv[kTile];
  __shared__ int32_t wpos[4][kMaxRad];  // per-wave counts, then next local places
  __shared__ int32_t delta[kMaxRad];    // global place minus local place, per digit
  __shared__ int tmp[4];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int rad = 1 << sp.dbits;
  const uint32_t dmask = (uint32_t)(rad - 1);
  const int64_t st = (int64_t)blockIdx.x / sp.tps, tile = (int64_t)blockIdx.x - st * sp.tps;
  const int64_t t0 = tile * kTile, t1 = std::min<int64_t>(sp.L, t0 + kTile);
  const int cnt = (int)(t1 - t0);
  // A. the events (wave w: rows w*kU .. w*kU + kU - 1 of the tile), the
  // digits' first global places, cleared counts
  uint32_t k[kU], v[kU];
#pragma unroll
  for (int u = 0; u < kU; u++) {
    const int64_t p = t0 + (int64_t)(wave * kU + u) * 64 + lane;
    const bool on = p < t1;
    uint32_t kf = 0u, vf = 0u;
    if (FIRST && on) first_pass_event(a, st, p, kf, vf);
    k[u] = on ? (FIRST ? kf : kin[st * sp.L + p]) : 0u;
    v[u] = on ? (FIRST ? vf : vin[st * sp.L + p]) : 0u;
  }
  const int per = rad > 256 ? rad / 256 : 1;
  int gs[kPer];
#pragma unroll
  for (int i = 0; i < kPer; i++) {
    const int d = tid * per + i;
    gs[i] = (i < per && d < rad) ? offs[(st * rad + d) * sp.tps + tile] : 0;
  }
  for (int i = tid; i < 4 * rad; i += 256) wpos[i / rad][i % rad] = 0;
  __syncthreads();
  // B. per-wave digit counts
#pragma unroll
  for (int u = 0; u < kU; u++)
    if (t0 + (int64_t)(wave * kU + u) * 64 + lane < t1) atomicAdd(&wpos[wave][(k[u] >> sp.shift) & dmask], 1);
  __syncthreads();
  // C. local places: thread tid owns digits tid*per .. tid*per + per - 1
  int cw[kPer][4];
  int tot = 0;
#pragma unroll
  for (int i = 0; i < kPer; i++) {
    const int d = tid * per + i;
#pragma unroll
    for (int w = 0; w < 4; w++) {
      cw[i][w] = (i < per && d < rad) ? wpos[w][d] : 0;
      tot += cw[i][w];
    }
  }
  int run = exsum::block_excl256(tot, tmp);  // (its barriers order every read above)
#pragma unroll
  for (int i = 0; i < kPer; i++) {
    const int d = tid * per + i;
    if (i < per && d < rad) {
      delta[d] = gs[i] - run;
#pragma unroll
      for (int w = 0; w < 4; w++) {
        wpos[w][d] = run;
        run += cw[i][w];
      }
    }
  }
  __syncthreads();
  // D. the local sort
  const uint64_t below = (uint64_t{1} << lane) - 1u;
#pragma unroll
  for (int u = 0; u < kU; u++) {
    const bool on = t0 + (int64_t)(wave * kU + u) * 64 + lane < t1;
    const uint32_t d = (k[u] >> sp.shift) & dmask;
    uint64_t peers = __ballot(on);
    for (int b = 0; b < sp.dbits; b++) {
      const uint64_t ones = __ballot((d >> b) & 1u);
      peers &= ((d >> b) & 1u) ? ones : ~ones;
    }
    if (on) {
      const int32_t lp = wpos[wave][d] + __popcll(peers & below);
      sk[lp] = k[u];
      sv[lp] = v[u];
      if ((peers >> lane) == 1u) wpos[wave][d] = lp + 1;  // the digit's last lane of the row
    }
  }
  __syncthreads();
  // E. out in local order
  for (int i = tid; i < cnt; i += 256) {
    const uint32_t kk = sk[i];
    const int32_t gp = delta[(kk >> sp.shift) & dmask] + i;
    kout[gp] = kk;
    vout[gp] = sv[i];
  }
}

// 2. slot segments.  A lane group takes the segments that start in its chunk
// of the sorted events (following each to its end, past the chunk if need
// be).  Event i of the sorted order belongs to stream i / L and names slot
// ks[i]; vs[i] is its position t*(W+R) + j in the stream (j < W: write rank
// j, else read rank j - W).
template <int LPR, bool VBF16>
__global__ void __launch_bounds__(256) sdm_tp_segments_kernel(TpArgs a, const uint32_t* ks,
                                                              const uint32_t* vs,
                                                              float* readbuf) {
#pragma clang fp contract(off)
  const int lane = threadIdx.x & 63;
  const int l = lane % LPR;
  const int64_t grp = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) / LPR;
  const int WR = a.W + a.R;
  const int64_t L = (int64_t)a.T * WR;
  const int64_t n = (int64_t)a.S * L;
  int64_t i = grp * kSegChunk;
  if (i >= n) return;  // no cross-lane operation follows
  const int64_t end = std::min(n, i + kSegChunk);
  const int c0 = 4 * l;
  // skip the tail of a segment that started in the previous chunk
  while (i < end && i % L != 0 && ks[i] == ks[i - 1]) i++;
  if (i >= end) return;
  int64_t st = i / L;
  int64_t send = (st + 1) * L;  // where the stream's events end
  auto rowp = [&](int64_t s, uint32_t slot) {
    return a.M + (s * a.N + (int64_t)slot) * a.d_v + c0;
  };
  // slots and payloads two events ahead: the next segment's row and this
  // event's gates and v are in flight together
  uint32_t scur = ks[i];
  uint32_t pj = vs[i];
  bool more1 = i + 1 < n;
  uint32_t k1 = more1 ? ks[i + 1] : 0u;
  uint32_t p1 = more1 ? vs[i + 1] : 0u;
  float* row = rowp(st, scur);
  float4 m = *reinterpret_cast<const float4*>(row);
  bool dirty = false;
  for (int64_t j = i;; j++) {
    const bool more2 = j + 2 < n;
    const uint32_t k2 = more2 ? ks[j + 2] : 0u;
    const uint32_t p2 = more2 ? vs[j + 2] : 0u;
    const bool cross = j + 1 == send;                      // event j+1 opens the next stream
    const bool ends = !more1 || cross || k1 != scur;      // event j closes its segment
    const bool next_here = more1 && ends && j + 1 < end;  // and the next one is ours
    const int64_t st1 = cross ? st + 1 : st;
    float* row1 = next_here ? rowp(st1, k1) : row;
    const float4 mnext = *reinterpret_cast<const float4*>(row1);  // (row itself if unused)
    const bool ign = (pj & kIgnored) != 0u;
    const uint32_t pos = pj & ~kIgnored;
    const int t = (int)(pos / WR), r = (int)(pos - (uint32_t)t * WR);
    const int64_t tok = st * a.T + t;
    if (r < a.W) {
      if (!ign) {
        const float c = a.beta[tok] * a.wwt[tok * a.W + r];
        const float omc = 1.0f - c;
        const float al = a.alpha[tok];
        const float4 v = load_v4(a.v, VBF16, tok * a.d_v + c0);
        m.x = omc * (al * m.x) + c * v.x;
        m.y = omc * (al * m.y) + c * v.y;
        m.z = omc * (al * m.z) + c * v.z;
        m.w = omc * (al * m.w) + c * v.w;
        dirty = true;
      }
    } else {
      *reinterpret_cast<float4*>(readbuf + (tok * a.R + (r - a.W)) * a.d_v + c0) =
          ign ? make_float4(0.f, 0.f, 0.f, 0.f) : m;
    }
    if (ends) {
      if (dirty) *reinterpret_cast<float4*>(row) = m;
      if (!next_here) break;  // no more events, or the next segment is the next chunk's
      scur = k1;
      if (cross) {
        st = st1;
        send += L;
      }
      row = row1;
      m = mnext;
      dirty = false;
    }
    pj = p1;
    more1 = more2;
    k1 = k2;
    p1 = p2;
  }
}

// 3. out[tok] = sum over r ascending of rwt[tok][r] * readbuf[tok][r], one
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

struct SortPlan {
  int npass, dbits;
  int64_t L, tps, nh;  // events per stream, tiles per stream, digit counts
};

SortPlan sort_plan(int S, int T, int64_t N, int W, int R) {
  SortPlan q{};
  const int nbits = std::max(1, host_bits(N));
  q.npass = (nbits + kMaxDigit - 1) / kMaxDigit;
  q.dbits = (nbits + q.npass - 1) / q.npass;
  q.L = (int64_t)T * (W + R);
  q.tps = (q.L + kTile - 1) / kTile;
  q.nh = (int64_t)S * (int64_t{1} << q.dbits) * q.tps;
  return q;
}

}  // namespace

bool tp_sizes_ok(int S, int T, int W, int R) {
  // positions and sorted places are int32
  return (int64_t)S * T * (W + R) < (int64_t{1} << 31);
}

size_t tp_workspace_bytes(int S, int T, int64_t N, int d_v, int W, int R) {
  const SortPlan q = sort_plan(S, T, N, W, R);
  const int64_t n = (int64_t)S * q.L;
  return 4 * align256(n * 4) + align256((size_t)(q.nh + 1) * 4) +
         align256((size_t)exsum::blocks(q.nh + 1) * 4) +
         align256((size_t)S * T * R * d_v * 4);
}

hipError_t launch_scan_tp(const TpArgs& a, bool vbf16, void* ws, hipStream_t stream) {
  const SortPlan q = sort_plan(a.S, a.T, a.N, a.W, a.R);
  const int64_t n = (int64_t)a.S * q.L;
  if (n == 0) return hipSuccess;
  unsigned char* p = static_cast<unsigned char*>(ws);
  uint32_t* kbuf[2];
  uint32_t* vbuf[2];
  for (int b = 0; b < 2; b++) {
    kbuf[b] = reinterpret_cast<uint32_t*>(p);
    p += align256(n * 4);
    vbuf[b] = reinterpret_cast<uint32_t*>(p);
    p += align256(n * 4);
  }
  int32_t* gh = reinterpret_cast<int32_t*>(p);
  p += align256((size_t)(q.nh + 1) * 4);
  int32_t* bsum = reinterpret_cast<int32_t*>(p);
  p += align256((size_t)exsum::blocks(q.nh + 1) * 4);
  float* readbuf = reinterpret_cast<float*>(p);

  // 1. the slot sort, pass k into buffer k % 2
  const int64_t ntiles = (int64_t)a.S * q.tps;
  const unsigned tgrid = (unsigned)((ntiles + 3) / 4);  // counts: a wave per tile
  hipError_t e;
  for (int k = 0; k < q.npass; k++) {
    const SortPass sp{q.L, q.tps, k * q.dbits, q.dbits};
    const uint32_t* kin = k ? kbuf[(k - 1) & 1] : nullptr;
    const uint32_t* vin = k ? vbuf[(k - 1) & 1] : nullptr;
    if (k == 0)
      hipLaunchKernelGGL(sdm_tp_hist_kernel<true>, dim3(tgrid), dim3(256), 0, stream, a, sp,
                         kin, gh);
    else
      hipLaunchKernelGGL(sdm_tp_hist_kernel<false>, dim3(tgrid), dim3(256), 0, stream, a, sp,
                         kin, gh);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if ((e = exsum::run(gh, q.nh, bsum, stream)) != hipSuccess) return e;
    if (k == 0)
      hipLaunchKernelGGL(sdm_tp_scatter_kernel<true>, dim3((unsigned)ntiles), dim3(256), 0,
                         stream, a, sp, kin, vin, gh, kbuf[k & 1], vbuf[k & 1]);
    else
      hipLaunchKernelGGL(sdm_tp_scatter_kernel<false>, dim3((unsigned)ntiles), dim3(256), 0,
                         stream, a, sp, kin, vin, gh, kbuf[k & 1], vbuf[k & 1]);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  const uint32_t* ks = kbuf[(q.npass - 1) & 1];
  const uint32_t* vs = vbuf[(q.npass - 1) & 1];

  // 2. slot segments
  const int lpr = a.d_v / 4;
  const int64_t groups = (n + kSegChunk - 1) / kSegChunk;
  const int64_t threads = groups * lpr;
  const unsigned sgrid = (unsigned)((threads + 255) / 256);
#define SDM_TP_SEG(LPR_)                                                                      \
  if (lpr == LPR_) {                                                                          \
    if (vbf16)                                                                                \
      hipLaunchKernelGGL((sdm_tp_segments_kernel<LPR_, true>), dim3(sgrid), dim3(256), 0,     \
                         stream, a, ks, vs, readbuf);                                         \
    else                                                                                      \
      hipLaunchKernelGGL((sdm_tp_segments_kernel<LPR_, false>), dim3(sgrid), dim3(256), 0,    \
                         stream, a, ks, vs, readbuf);                                         \
  } else
  SDM_TP_SEG(4) SDM_TP_SEG(8) SDM_TP_SEG(16) SDM_TP_SEG(32) SDM_TP_SEG(64) {
    return hipErrorInvalidValue;
  }
#undef SDM_TP_SEG
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  // 3. read sums
  const int64_t nr = (int64_t)a.S * a.T * (a.d_v / 4);
  const int rgrid = (int)std::min<int64_t>((nr + 255) / 256, 65536);
  hipLaunchKernelGGL(sdm_tp_reduce_kernel, dim3(rgrid), dim3(256), 0, stream, a, readbuf);
  return hipGetLastError();
}

}  // namespace sdm
