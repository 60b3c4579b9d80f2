// Adjoint of product-key addressing, for gfx950: gradients of the slot weights
// to the projected queries and keys and to the sub-key tables.
//
// Forward ("Sparse Delta Memory", gist.science summaries of paper 2607.07386;
// Spanish page "Mecanismo Central" item 2): slot s = i*n_sub + j has score
// sigma = <x_1, C_1[i]> + <x_2, C_2[j]> (x_1, x_2 the halves of k' or q'), and the
// W write (R read) slots get softmax weights w over their scores.  The
// selection is piecewise constant, so with the slots held fixed:
//   dsigma_r = w_r * (dw_r - sum_u w_u dw_u)
//   dx_1 = sum_r dsigma_r C_1[i_r],   dx_2 = sum_r dsigma_r C_2[j_r]
//   dC_1[i] += sum_{r: i_r = i} dsigma_r x_1,   dC_2[j] likewise with x_2.
//
// One wave per (token, side): side 0 is the write set (k', dk'), side 1 the
// read set (q', dq').  The wave folds the dsigma of slots that share a sub-key
// row in a small LDS hash per half (row -> dsigma sum and the row's first
// event) and lists the distinct rows in the order of their first events.  The
// fold adds 64-bit fixed-point integers (every dsigma of the wave scaled by
// one power of two, so that 128 of them cannot overflow), so the order in
// which the lanes' atomic adds land cannot change the sum: it is the exact sum
// of the scaled values, rounded once back to fp32.  It
// gathers those rows 16 bytes a lane for dx, and writes one record per
// distinct row, (table row, token-side, dsigma sum), into fixed slots (unused
// slots get only a key, one that sorts last; their payload is never read).
//
// The table gradient is then a sum per table row over the records that name
// it.  A stable counting sort groups the records by row, keeping their
// (token, side, half) order inside a row: the keys of one head are its 2*n_sub
// sub-key rows, so each chunk of a stream's tokens counts them in an LDS
// histogram; one exclusive scan over (row, chunk) gives every chunk's first
// position per row; and one wave per chunk walks its groups in order, placing
// each record at its row's next position.  The records of one group name
// distinct rows, so that walk needs no atomics and its order is the input
// order.  One wave per table row then adds dsigma * x over its records in
// that order.  Every floating-point sum has a fixed order and the fold's
// atomics add integers, so dq', dk' and the sub-key gradient are the same bit
// for bit on every run.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "excl_sum.h"
#include "sdm_internal.h"

namespace sdm {

namespace {

constexpr int kWavesBwd = 8;  // waves per workgroup (4 tokens x 2 sides)
constexpr int kRedWaves = 4;  // waves per workgroup of the row sums
constexpr int kChunks = 1024;  // counting-sort chunks a launch aims for
constexpr int kStage = 1024;   // record slots of one scatter batch (256 threads x 4)


template <bool BF16>
__device__ __forceinline__ float elem(const void* p, int64_t i) {
  if constexpr (BF16) {
    return __uint_as_float((uint32_t) static_cast<const uint16_t*>(p)[i] << 16);
  } else {
    return static_cast<const float*>(p)[i];
  }
}

__device__ __forceinline__ float wave_sum(float x) {
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

// LDS hash of one half's rows for one wave: key row (-1 empty), the row's
// first event (lowest rank) and its dsigma sum in fixed point.
struct RowEnt {
  int32_t key;
  int32_t first;
  unsigned long long acc;  // two's complement sum of the scaled dsigma
};

// a distinct row of one half and its dsigma sum
struct RowSum {
  int32_t key;
  float sum;
};

// Fixed-point scale: with m = the wave's largest |dsigma| < 2^e, values are
// multiplied by 2^(54 - e), so each is below 2^54 in magnitude and a sum of
// at most 128 of them below 2^61.  The scaling is exact; rounding to an
// integer drops only bits below 2^-54 of m.
__device__ __forceinline__ int fixed_shift(float m) {
  if (!(m > 0.f)) return 0;
  int e;
  frexpf(m, &e);
  return 54 - e;
}

__device__ __forceinline__ unsigned long long to_fixed(float x, int sh) {
  return (unsigned long long)(long long)rint(ldexp((double)x, sh));
}

__device__ __forceinline__ float from_fixed(unsigned long long a, int sh) {
  return (float)ldexp((double)(long long)a, -sh);
}

// entries per half: a power of two >= 2k (k <= 128)
__host__ __device__ inline int row_table_size(int k) {
  int n = 16;
  while (n < 2 * k) n *= 2;
  return n;
}

// LDS of one wave: two row tables and the distinct-row list (16-byte multiple)
__host__ __device__ inline size_t wave_lds_bytes(int kmax) {
  const size_t b = (size_t)2 * row_table_size(kmax) * sizeof(RowEnt) + (size_t)kmax * sizeof(RowSum);
  return (b + 15) & ~(size_t)15;
}

template <bool BF16>
__global__ void __launch_bounds__(kWavesBwd * 64)
    sdm_score_bwd_kernel(ScoreBwdArgs a, uint32_t* __restrict__ rkey, uint64_t* __restrict__ rval,
                         int32_t* __restrict__ gcnt) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int n_sub = a.n_sub;
  const int kmax = a.W > a.R ? a.W : a.R;
  const int HT = row_table_size(kmax);
  // per wave: two row tables, then the distinct rows of a half (row, sum)
  RowEnt* tab = reinterpret_cast<RowEnt*>(smem + (size_t)wave * wave_lds_bytes(kmax));
  RowSum* dist = reinterpret_cast<RowSum*>(tab + 2 * HT);

  const int64_t unit = (int64_t)blockIdx.x * (kWavesBwd / 2) + (wave >> 1);  // stream-token
  const int side = wave & 1;
  if (unit >= (int64_t)a.S * a.T) return;  // wave-uniform; no barrier below
  const int st = (int)(unit / a.T);
  const int h = st % a.H;
  const int k = side ? a.R : a.W;
  const int32_t* idx = (side ? a.ridx : a.widx) + unit * k;
  const float* wt = (side ? a.rwt : a.wwt) + unit * k;
  const float* dw = (side ? a.drwt : a.dwwt) + unit * k;
  float* dx = (side ? a.dq : a.dk) + unit * a.d_k;
  const int dh = a.d_k / 2;

  // ---- softmax adjoint (k <= 128: two events per lane) ---------------------
  float ds[2], wv[2], gv[2];
  int32_t rowv[2][2];
  float sw = 0.f;
#pragma unroll
  for (int u = 0; u < 2; u++) {
    const int r = u * 64 + lane;
    const bool on = r < k;
    wv[u] = on ? wt[r] : 0.f;
    gv[u] = on ? dw[r] : 0.f;
    sw += wv[u] * gv[u];
    const int32_t s = on ? idx[r] : 0;
    rowv[0][u] = s / n_sub;
    rowv[1][u] = s - rowv[0][u] * n_sub;
  }
  const float dot = wave_sum(sw);
  float mx = 0.f;
#pragma unroll
  for (int u = 0; u < 2; u++) {
    ds[u] = wv[u] * (gv[u] - dot);
    mx = fmaxf(mx, fabsf(ds[u]));
  }
  for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
  const int sh = fixed_shift(mx);

  // ---- fold events that share a row (per half) ----------------------------
  for (int i = lane; i < 2 * HT; i += 64) tab[i] = RowEnt{-1, 0x7fffffff, 0ull};
  wave_lds_sync();
#pragma unroll
  for (int u = 0; u < 2; u++) {
    const int r = u * 64 + lane;
    if (r < k) {
#pragma unroll
      for (int half = 0; half < 2; half++) {
        const int32_t row = rowv[half][u];
        RowEnt* t = tab + half * HT;
        int p = (int)((uint32_t)row * 2654435761u >> 8) & (HT - 1);
        while (true) {
          const int32_t old = atomicCAS(&t[p].key, -1, row);
          if (old == -1 || old == row) break;
          p = (p + 1) & (HT - 1);
        }
        atomicMin(&t[p].first, r);
        atomicAdd(&t[p].acc, to_fixed(ds[u], sh));
      }
    }
  }
  wave_lds_sync();

  // ---- per half: distinct rows in rank order, then dx and the table gradient
  const int64_t cbase = (int64_t)h * 2 * n_sub * dh;
  const uint64_t below = (1ull << lane) - 1ull;
  for (int half = 0; half < 2; half++) {
    const RowEnt* t = tab + half * HT;
    int nd = 0;
#pragma unroll
    for (int u = 0; u < 2; u++) {
      const int r = u * 64 + lane;
      float sum = 0.f;
      bool own = false;
      if (r < k) {
        int p = (int)((uint32_t)rowv[half][u] * 2654435761u >> 8) & (HT - 1);
        while (t[p].key != rowv[half][u]) p = (p + 1) & (HT - 1);
        own = t[p].first == r;
        sum = from_fixed(t[p].acc, sh);
      }
      const uint64_t bal = __ballot(own);
      if (own) dist[nd + __popcll(bal & below)] = RowSum{rowv[half][u], sum};
      nd += __popcll(bal);
    }
    wave_lds_sync();
    const int64_t hbase = cbase + (int64_t)half * n_sub * dh;
    // dx = sum over the distinct rows of dsigma * C[row]: each lane loads 16
    // bytes of a row, RPI rows per load instruction (LRp lanes per row, the
    // row's LR chunks rounded up to a power of two), up to NI instructions in
    // flight; each lane sums its rows in order, then the row slots are added
    // by a butterfly, so the order is fixed
    constexpr int EL = BF16 ? 8 : 4;  // elements per 16-byte chunk
    constexpr int NI = 8;
    const int LR = dh / EL;
    int LRp = 1;
    while (LRp < LR) LRp <<= 1;
    const int RPI = 64 / LRp;
    const int sub = lane & (LRp - 1), slot = lane / LRp;
    const bool lon = sub < LR;
    const unsigned char* cb = static_cast<const unsigned char*>(a.subkeys) +
                              (hbase + (int64_t)sub * EL) * (BF16 ? 2 : 4);
    const int64_t rstride = (int64_t)dh * (BF16 ? 2 : 4);
    float acc[EL];
#pragma unroll
    for (int e = 0; e < EL; e++) acc[e] = 0.f;
    {
      // this half's records, group ts*2 + half: the distinct rows in the order
      // of their first events, and how many there are
      const int64_t ts = unit * 2 + side;
      const int64_t r0 = (ts * 2 + half) * kmax;
      const uint32_t kbase = (uint32_t)((h * 2 + half) * n_sub);
      for (int j = lane; j < nd; j += 64) {
        rkey[r0 + j] = kbase + (uint32_t)dist[j].key;
        rval[r0 + j] = ((uint64_t)ts << 32) | __float_as_uint(dist[j].sum);
      }
      if (lane == 0) gcnt[ts * 2 + half] = nd;
    }
    for (int b0 = 0; b0 < nd; b0 += NI * RPI) {
      uint4 ch[NI];
      float gg[NI];
#pragma unroll
      for (int i = 0; i < NI; i++) {
        const int r = b0 + i * RPI + slot;
        const bool ok = lon && r < nd;
        const int32_t row = ok ? dist[r].key : 0;  // row 0 keeps the address inside the table
        gg[i] = ok ? dist[r].sum : 0.f;
        ch[i] = *reinterpret_cast<const uint4*>(cb + (int64_t)row * rstride);
      }
#pragma unroll
      for (int i = 0; i < NI; i++) {
        const uint32_t w[4] = {ch[i].x, ch[i].y, ch[i].z, ch[i].w};
#pragma unroll
        for (int e = 0; e < EL; e++) {
          float f;
          if constexpr (BF16)
            f = __uint_as_float((e & 1) ? (w[e >> 1] & 0xffff0000u) : (w[e >> 1] << 16));
          else
            f = __uint_as_float(w[e]);
          acc[e] += gg[i] * f;
        }
      }
    }
    for (int o = LRp; o < 64; o <<= 1) {
#pragma unroll
      for (int e = 0; e < EL; e++) acc[e] += __shfl_xor(acc[e], o);
    }
    if (slot == 0 && lon) {
      float* d = dx + half * dh + sub * EL;
#pragma unroll
      for (int e = 0; e < EL; e += 4)
        *reinterpret_cast<float4*>(d + e) = make_float4(acc[e], acc[e + 1], acc[e + 2], acc[e + 3]);
    }
    wave_lds_sync();  // the distinct list is rebuilt for the next half
  }
}

// ---- stable counting sort of the records by table row ------------------------
// Groups g = (token-side) * 2 + half hold gcnt[g] records at [g*kmax, ...), all
// naming distinct rows of one head (keys h*2*n_sub .. +2*n_sub).  A chunk is
// up to CH tokens of one stream (4 groups per token; CH is chosen so that a
// launch has about kChunks chunks, each walked by one wave), and cnt holds, for
// each head h, local key l and chunk c of that head (chunks of streams
// b*H + h, ordered by b then position in the stream), the records of key l in
// chunk c at cnt[(h*2*n_sub + l) * BnC + c]: its exclusive scan is the first
// position of every (key, chunk) in the sorted list.
struct SortGeom {
  int T, H, n_sub, kmax, CH, nC, BnC;
};

// chunk (blockIdx.x, stream blockIdx.y): its head, its column in cnt, its groups
__device__ __forceinline__ void chunk_of(const SortGeom& q, int& h, int& col, int64_t& g0,
                                         int64_t& g1) {
  const int st = blockIdx.y, tc = blockIdx.x;
  h = st % q.H;
  col = (st / q.H) * q.nC + tc;
  const int64_t t0 = (int64_t)st * q.T + (int64_t)tc * q.CH;
  const int64_t t1 = std::min((int64_t)st * q.T + q.T, t0 + q.CH);
  g0 = t0 * 4;
  g1 = t1 * 4;
}

__global__ void __launch_bounds__(256) sdm_bwd_count_kernel(SortGeom q,
                                                            const uint32_t* __restrict__ rkey,
                                                            const int32_t* __restrict__ gcnt,
                                                            int32_t* __restrict__ cnt) {
  extern __shared__ int32_t hist[];  // [2*n_sub]
  int h, col;
  int64_t g0, g1;
  chunk_of(q, h, col, g0, g1);
  const int nloc = 2 * q.n_sub;
  const uint32_t kb = (uint32_t)h * nloc;
  for (int l = threadIdx.x; l < nloc; l += 256) hist[l] = 0;
  __syncthreads();
  // record slots in batches of kU per thread: every group count of a batch
  // is loaded before any key, and every key before any count is taken
  constexpr int kU = 8;
  const int64_t nslot = (g1 - g0) * q.kmax;
  for (int64_t base = threadIdx.x; base < nslot; base += 256 * kU) {
    int gc[kU];
    uint32_t kk[kU];
#pragma unroll
    for (int u = 0; u < kU; u++) {
      const int64_t i = base + u * 256;
      gc[u] = i < nslot ? gcnt[g0 + i / q.kmax] : 0;
    }
#pragma unroll
    for (int u = 0; u < kU; u++) {
      const int64_t i = base + u * 256;
      const int64_t g = g0 + i / q.kmax;
      const int j = (int)(i - (g - g0) * q.kmax);
      kk[u] = (i < nslot && j < gc[u]) ? rkey[g * q.kmax + j] : 0xffffffffu;
    }
#pragma unroll
    for (int u = 0; u < kU; u++)
      if (kk[u] != 0xffffffffu) atomicAdd(&hist[kk[u] - kb], 1);
  }
  __syncthreads();
  for (int l = threadIdx.x; l < nloc; l += 256)
    cnt[((int64_t)h * nloc + l) * q.BnC + col] = hist[l];
}

// Scatter: the chunk's groups go in batches of up to 32, in order.  In a
// batch, every record sets its group's bit in an LDS mask of its row (the
// records of one group name distinct rows, and OR does not depend on the
// order it is applied in); a record's position is then its row's next
// position plus the number of earlier groups of the batch that name the row;
// and the record of the row's last group in the batch advances that next
// position past the batch.  So every record lands where a walk in group
// order would put it, with no serial step.  The next batch's records are
// loaded while a batch is placed, and its group counts one batch earlier.
__global__ void __launch_bounds__(256) sdm_bwd_scatter_kernel(
    SortGeom q, const uint32_t* __restrict__ rkey, const uint64_t* __restrict__ rval,
    const int32_t* __restrict__ gcnt, const int32_t* __restrict__ offs,
    uint64_t* __restrict__ vout) {
  extern __shared__ int32_t lds[];
  const int nloc = 2 * q.n_sub;
  int32_t* run = lds;                                     // [nloc] next position of each row
  uint32_t* mask = reinterpret_cast<uint32_t*>(lds + nloc);  // [nloc] groups of the batch
  int h, col;
  int64_t g0, g1;
  chunk_of(q, h, col, g0, g1);
  const uint32_t kb = (uint32_t)h * nloc;
  const int tid = threadIdx.x;
  {
    // every first position is loaded before any is stored (one round trip)
    constexpr int kU = 8;
    for (int l0 = tid; l0 < nloc; l0 += 256 * kU) {
      int v[kU];
#pragma unroll
      for (int u = 0; u < kU; u++) {
        const int l = l0 + u * 256;
        v[u] = l < nloc ? offs[((int64_t)h * nloc + l) * q.BnC + col] : 0;
      }
#pragma unroll
      for (int u = 0; u < kU; u++)
        if (l0 + u * 256 < nloc) {
          run[l0 + u * 256] = v[u];
          mask[l0 + u * 256] = 0u;
        }
    }
  }
  const int sg = std::max(1, std::min(32, kStage / q.kmax));  // groups per batch
  constexpr int kU = kStage / 256;  // record slots per thread per batch
  // slot i = tid + u*256 of a batch is record j = i % kmax of group i / kmax
  auto counts = [&](int64_t gs, int (&gc)[kU]) {
    const int nrec = (int)std::min<int64_t>(sg, g1 - gs) * q.kmax;
#pragma unroll
    for (int u = 0; u < kU; u++) {
      const int i = tid + u * 256;
      gc[u] = (gs < g1 && i < nrec) ? gcnt[gs + i / q.kmax] : 0;
    }
  };
  auto records = [&](int64_t gs, const int (&gc)[kU], uint32_t (&kk)[kU], uint64_t (&vv)[kU]) {
#pragma unroll
    for (int u = 0; u < kU; u++) {
      const int i = tid + u * 256;
      const int gq = i / q.kmax, j = i - gq * q.kmax;
      const bool on = j < gc[u];  // gc is 0 past the batch
      kk[u] = on ? rkey[(gs + gq) * q.kmax + j] : 0xffffffffu;
      vv[u] = on ? rval[(gs + gq) * q.kmax + j] : 0ull;
    }
  };
  int gcn[kU], gcnn[kU];
  uint32_t kn[kU];
  uint64_t vn[kU];
  counts(g0, gcn);
  records(g0, gcn, kn, vn);
  counts(g0 + sg, gcnn);
  __syncthreads();  // run and mask are filled
  for (int64_t gs = g0; gs < g1; gs += sg) {
    uint32_t kc[kU];
    uint64_t vc[kU];
#pragma unroll
    for (int u = 0; u < kU; u++) kc[u] = kn[u], vc[u] = vn[u];
    // the next batch in flight
    records(gs + sg, gcnn, kn, vn);
    counts(gs + 2 * sg, gcnn);
    // 1. groups naming each row
#pragma unroll
    for (int u = 0; u < kU; u++)
      if (kc[u] != 0xffffffffu) atomicOr(&mask[kc[u] - kb], 1u << ((tid + u * 256) / q.kmax));
    __syncthreads();
    // 2. positions
    uint32_t m[kU];
#pragma unroll
    for (int u = 0; u < kU; u++) {
      m[u] = 0u;
      if (kc[u] != 0xffffffffu) {
        const int loc = (int)(kc[u] - kb);
        const int gq = (tid + u * 256) / q.kmax;
        m[u] = mask[loc];
        vout[run[loc] + __popc(m[u] & ((1u << gq) - 1u))] = vc[u];
      }
    }
    __syncthreads();
    // 3. the row's last group of the batch moves its next position on
#pragma unroll
    for (int u = 0; u < kU; u++) {
      if (kc[u] != 0xffffffffu) {
        const int gq = (tid + u * 256) / q.kmax;
        if ((m[u] >> gq) == 1u) {
          const int loc = (int)(kc[u] - kb);
          run[loc] += __popc(m[u]);
          mask[loc] = 0u;
        }
      }
    }
    __syncthreads();
  }
}

// Table gradient: one wave per table row (h, half, row) adds dsigma * x of
// every record of that row, in record order, to dsub (which accumulates).
// Each lane loads 16 bytes of a record's x half, LRp lanes per record (the
// row's chunks rounded up to a power of two), RPI records per load
// instruction and NI instructions in flight; the next batch's records are
// read while the current one is summed.  Lane slot s sums records s, s + RPI,
// ... in order, then the slots are added by a butterfly: a fixed order.
template <bool BF16>
__global__ void __launch_bounds__(kRedWaves * 64)
    sdm_score_bwd_reduce_kernel(ScoreBwdArgs a, const uint64_t* __restrict__ rval,
                                const int32_t* __restrict__ offs, int BnC) {
  constexpr int EL = BF16 ? 8 : 4;  // elements per 16-byte chunk
  constexpr int NI = 4;
  const int lane = threadIdx.x & 63;
  const int64_t key = (int64_t)blockIdx.x * kRedWaves + (threadIdx.x >> 6);
  const int64_t nkeys = (int64_t)a.H * 2 * a.n_sub;
  if (key >= nkeys) return;  // wave-uniform; no barrier follows
  const int i0 = offs[key * BnC], i1 = offs[(key + 1) * BnC];
  if (i1 <= i0) return;
  const int dh = a.d_k / 2;
  const int half = (int)((key / a.n_sub) & 1);
  const int LR = dh / EL;
  int LRp = 1;
  while (LRp < LR) LRp <<= 1;
  const int RPI = 64 / LRp;
  const int sub = lane & (LRp - 1), slot = lane / LRp;
  const bool lon = sub < LR;
  const int64_t cofs = (int64_t)half * dh + (int64_t)sub * EL;  // element offset in a d_k row
  const int step = NI * RPI;
  float acc[EL];
#pragma unroll
  for (int e = 0; e < EL; e++) acc[e] = 0.f;
  uint64_t vn[NI];
#pragma unroll
  for (int i = 0; i < NI; i++) {
    const int r = i0 + i * RPI + slot;
    vn[i] = rval[r < i1 ? r : i0];
  }
  for (int b = i0; b < i1; b += step) {
    uint64_t v[NI];
#pragma unroll
    for (int i = 0; i < NI; i++) v[i] = vn[i];
    uint4 ch[NI];
#pragma unroll
    for (int i = 0; i < NI; i++) {
      const int64_t ts = (int64_t)(v[i] >> 32);
      const unsigned char* xin = static_cast<const unsigned char*>((ts & 1) ? a.qp : a.kp);
      const int64_t el = (ts >> 1) * a.d_k + (lon ? cofs : 0);
      ch[i] = *reinterpret_cast<const uint4*>(xin + el * (BF16 ? 2 : 4));
    }
#pragma unroll
    for (int i = 0; i < NI; i++) {  // the next batch's records
      const int r = b + step + i * RPI + slot;
      vn[i] = rval[r < i1 ? r : i0];
    }
#pragma unroll
    for (int i = 0; i < NI; i++) {
      const int r = b + i * RPI + slot;
      const float g = (lon && r < i1) ? __uint_as_float((uint32_t)v[i]) : 0.f;
      const uint32_t w[4] = {ch[i].x, ch[i].y, ch[i].z, ch[i].w};
#pragma unroll
      for (int e = 0; e < EL; e++) {
        float f;
        if constexpr (BF16)
          f = __uint_as_float((e & 1) ? (w[e >> 1] & 0xffff0000u) : (w[e >> 1] << 16));
        else
          f = __uint_as_float(w[e]);
        acc[e] += g * f;
      }
    }
  }
  for (int o = LRp; o < 64; o <<= 1) {
#pragma unroll
    for (int e = 0; e < EL; e++) acc[e] += __shfl_xor(acc[e], o);
  }
  if (slot == 0 && lon) {
    float* d = a.dsub + key * dh + sub * EL;
#pragma unroll
    for (int e = 0; e < EL; e += 4) {
      float4 t = *reinterpret_cast<float4*>(d + e);
      t.x += acc[e];
      t.y += acc[e + 1];
      t.z += acc[e + 2];
      t.w += acc[e + 3];
      *reinterpret_cast<float4*>(d + e) = t;
    }
  }
}

size_t align256(size_t x) { return (x + 255) & ~size_t{255}; }

SortGeom sort_geom(int S, int T, int H, int n_sub, int W, int R) {
  SortGeom q;
  q.T = T;
  q.H = H;
  q.n_sub = n_sub;
  q.kmax = W > R ? W : R;
  const int64_t per = ((int64_t)S * T + kChunks - 1) / kChunks;
  q.CH = (int)std::min<int64_t>(std::max<int64_t>(per, 32), 1024);
  q.nC = (T + q.CH - 1) / q.CH;
  q.BnC = (S / H) * q.nC;
  return q;
}

size_t scatter_lds_bytes(const SortGeom& q) { return (size_t)2 * (2 * q.n_sub) * 4; }

}  // namespace

size_t score_bwd_lds_bytes(int kmax) { return (size_t)kWavesBwd * wave_lds_bytes(kmax); }

int64_t score_bwd_records(int S, int T, int W, int R) {
  return (int64_t)S * T * 4 * (W > R ? W : R);  // (token, side, half) x kmax
}

// records (keys, payloads, sorted payloads), group counts, the (row, chunk)
// counts and their scan, and the scan's block sums
size_t score_bwd_workspace_bytes(int S, int T, int H, int n_sub, int W, int R) {
  const int64_t n = score_bwd_records(S, T, W, R);
  const SortGeom q = sort_geom(S, T, H, n_sub, W, R);
  const int64_t M = (int64_t)H * 2 * n_sub * q.BnC;
  return align256((size_t)n * 4) + 2 * align256((size_t)n * 8) +
         align256((size_t)S * T * 4 * 4) + align256((size_t)(M + 1) * 4) +
         align256((size_t)exsum::blocks(M) * 4);
}

hipError_t launch_score_bwd(const ScoreBwdArgs& a, bool bf16, void* ws, hipStream_t stream) {
  const int64_t units = (int64_t)a.S * a.T;
  if (units == 0) return hipSuccess;
  const int64_t n = score_bwd_records(a.S, a.T, a.W, a.R);
  const SortGeom q = sort_geom(a.S, a.T, a.H, a.n_sub, a.W, a.R);
  const int64_t nkeys = (int64_t)a.H * 2 * a.n_sub;
  const int64_t M = nkeys * q.BnC;
  unsigned char* p = static_cast<unsigned char*>(ws);
  uint32_t* rkey = reinterpret_cast<uint32_t*>(p);
  p += align256((size_t)n * 4);
  uint64_t* rval = reinterpret_cast<uint64_t*>(p);
  p += align256((size_t)n * 8);
  uint64_t* vout = reinterpret_cast<uint64_t*>(p);
  p += align256((size_t)n * 8);
  int32_t* gcnt = reinterpret_cast<int32_t*>(p);
  p += align256((size_t)units * 4 * 4);
  int32_t* offs = reinterpret_cast<int32_t*>(p);  // counts, then their exclusive scan
  p += align256((size_t)(M + 1) * 4);
  int32_t* bsum = reinterpret_cast<int32_t*>(p);

  // 1. per (token, side): dsigma, dx, one record per distinct table row
  const int64_t grid = (units + kWavesBwd / 2 - 1) / (kWavesBwd / 2);
  const size_t lds = score_bwd_lds_bytes(a.W > a.R ? a.W : a.R);
  auto k = bf16 ? sdm_score_bwd_kernel<true> : sdm_score_bwd_kernel<false>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k, dim3((unsigned)grid), dim3(kWavesBwd * 64), lds, stream, a, rkey, rval,
                     gcnt);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // 2. records grouped by table row, in group order inside a row: counts per
  // (row, chunk), their exclusive scan, then the scatter
  const dim3 cgrid((unsigned)q.nC, (unsigned)a.S);
  hipLaunchKernelGGL(sdm_bwd_count_kernel, cgrid, dim3(256), (size_t)2 * a.n_sub * 4, stream, q,
                     rkey, gcnt, offs);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((e = exsum::run(offs, M, bsum, stream)) != hipSuccess) return e;
  const size_t slds = scatter_lds_bytes(q);
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(sdm_bwd_scatter_kernel),
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)slds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(sdm_bwd_scatter_kernel, cgrid, dim3(256), slds, stream, q, rkey, rval, gcnt,
                     offs, vout);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // 3. one wave per table row
  const unsigned rgrid = (unsigned)((nkeys + kRedWaves - 1) / kRedWaves);
  if (bf16)
    hipLaunchKernelGGL(sdm_score_bwd_reduce_kernel<true>, dim3(rgrid), dim3(kRedWaves * 64), 0,
                       stream, a, vout, offs, q.BnC);
  else
    hipLaunchKernelGGL(sdm_score_bwd_reduce_kernel<false>, dim3(rgrid), dim3(kRedWaves * 64), 0,
                       stream, a, vout, offs, q.BnC);
  return hipGetLastError();
}

}  // namespace sdm
