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
// event) and lists the distinct rows in the order of their first events.  It
// gathers those rows 16 bytes a lane for dx, and writes one record per
// distinct row, (table row, token-side, dsigma sum), into fixed slots (unused
// slots get only a key, one that sorts last; their payload is never read).
//
// The table gradient is then a sum per table row over the records that name
// it.  A radix sort (rocPRIM, stable) groups the records by row, keeping
// their slot order inside a row, and one wave per table row adds
// dsigma * x over its records in that order.  Every sum has a fixed order, so
// dq', dk' and the sub-key gradient are the same bit for bit on every run,
// and nothing is accumulated with atomics.
#include <hip/hip_runtime.h>
#include <rocprim/device/device_radix_sort.hpp>
#include <stdint.h>

#include "sdm_internal.h"

namespace sdm {

namespace {

constexpr int kWavesBwd = 8;  // waves per workgroup (4 tokens x 2 sides)
constexpr uint32_t kBwdPad = 0xffffffffu;  // key of an unused record slot (sorts last)
constexpr int kRedWaves = 4;               // waves per workgroup of the row sums

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
// first event (lowest rank) and its dsigma sum.
struct RowEnt {
  int32_t key;
  int32_t first;
  float sum;
};

// entries per half: a power of two >= 2k (k <= 128)
__host__ __device__ inline int row_table_size(int k) {
  int n = 16;
  while (n < 2 * k) n *= 2;
  return n;
}

template <bool BF16>
__global__ void __launch_bounds__(kWavesBwd * 64)
    sdm_score_bwd_kernel(ScoreBwdArgs a, uint32_t* __restrict__ rkey, uint64_t* __restrict__ rval) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int n_sub = a.n_sub;
  const int kmax = a.W > a.R ? a.W : a.R;
  const int HT = row_table_size(kmax);
  // per wave: two row tables, then the distinct rows of a half (row, sum)
  RowEnt* tab = reinterpret_cast<RowEnt*>(smem) + (size_t)wave * (2 * HT + kmax);
  RowEnt* dist = tab + 2 * HT;

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
#pragma unroll
  for (int u = 0; u < 2; u++) ds[u] = wv[u] * (gv[u] - dot);

  // ---- fold events that share a row (per half) ----------------------------
  for (int i = lane; i < 2 * HT; i += 64) tab[i] = RowEnt{-1, 0x7fffffff, 0.f};
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
        atomicAdd(&t[p].sum, ds[u]);
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
        sum = t[p].sum;
      }
      const uint64_t bal = __ballot(own);
      if (own) dist[nd + __popcll(bal & below)] = RowEnt{rowv[half][u], 0, sum};
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
      // this half's records: distinct rows in the order of their first
      // events, then padding keys up to kmax
      const int64_t ts = unit * 2 + side;
      const int64_t r0 = (ts * 2 + half) * kmax;
      const uint32_t kbase = (uint32_t)((h * 2 + half) * n_sub);
      for (int j = lane; j < kmax; j += 64) {
        const bool on = j < nd;
        rkey[r0 + j] = on ? kbase + (uint32_t)dist[j].key : kBwdPad;
        if (on) rval[r0 + j] = ((uint64_t)ts << 32) | __float_as_uint(dist[j].sum);
      }
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

// Record boundaries: after the sort, rows [start, end) of the record list hold
// table row key.  Rows no record names keep start = end = 0.
__global__ void __launch_bounds__(256) sdm_bwd_bounds_clear(int32_t* bounds, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    bounds[i] = 0;
}

__global__ void __launch_bounds__(256) sdm_bwd_bounds_kernel(const uint32_t* __restrict__ key,
                                                             int64_t n, uint32_t nkeys,
                                                             int32_t* __restrict__ bounds) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    const uint32_t k = key[i];
    if (k >= nkeys) continue;  // padding (sorted after every real key)
    if (i == 0 || key[i - 1] != k) bounds[2 * (int64_t)k] = (int32_t)i;
    if (i == n - 1 || key[i + 1] != k) bounds[2 * (int64_t)k + 1] = (int32_t)(i + 1);
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
                                const int32_t* __restrict__ bounds) {
  constexpr int EL = BF16 ? 8 : 4;  // elements per 16-byte chunk
  constexpr int NI = 4;
  const int lane = threadIdx.x & 63;
  const int64_t key = (int64_t)blockIdx.x * kRedWaves + (threadIdx.x >> 6);
  const int64_t nkeys = (int64_t)a.H * 2 * a.n_sub;
  if (key >= nkeys) return;  // wave-uniform; no barrier follows
  const int i0 = bounds[2 * key], i1 = bounds[2 * key + 1];
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

int bits_for(int64_t n) {  // bits to hold 0 .. n-1
  int b = 0;
  while ((int64_t{1} << b) < n) b++;
  return b;
}

size_t align256(size_t x) { return (x + 255) & ~size_t{255}; }

// rocPRIM's scratch for n pairs (a query; nothing runs)
size_t bwd_sort_temp_bytes(int64_t n, int end_bit) {
  size_t bytes = 0;
  const hipError_t e =
      rocprim::radix_sort_pairs(nullptr, bytes, (const uint32_t*)nullptr, (uint32_t*)nullptr,
                                (const uint64_t*)nullptr, (uint64_t*)nullptr, (size_t)n, 0,
                                (unsigned)end_bit);
  return e == hipSuccess ? bytes : SIZE_MAX / 4;  // an unmet size rather than a wrong one
}

}  // namespace

size_t score_bwd_lds_bytes(int kmax) {
  return (size_t)kWavesBwd * (2 * row_table_size(kmax) + kmax) * sizeof(RowEnt);
}

int64_t score_bwd_records(int S, int T, int W, int R) {
  return (int64_t)S * T * 4 * (W > R ? W : R);  // (token, side, half) x kmax
}

size_t score_bwd_workspace_bytes(int S, int T, int H, int n_sub, int W, int R) {
  const int64_t n = score_bwd_records(S, T, W, R);
  const int64_t nkeys = (int64_t)H * 2 * n_sub;
  const int end_bit = bits_for(nkeys + 1);
  return 2 * align256((size_t)n * 4) + 2 * align256((size_t)n * 8) +
         align256((size_t)nkeys * 8) + align256(bwd_sort_temp_bytes(n, end_bit));
}

hipError_t launch_score_bwd(const ScoreBwdArgs& a, bool bf16, void* ws, hipStream_t stream) {
  const int64_t units = (int64_t)a.S * a.T;
  if (units == 0) return hipSuccess;
  const int64_t n = score_bwd_records(a.S, a.T, a.W, a.R);
  const int64_t nkeys = (int64_t)a.H * 2 * a.n_sub;
  const int end_bit = bits_for(nkeys + 1);
  unsigned char* p = static_cast<unsigned char*>(ws);
  uint32_t* k_in = reinterpret_cast<uint32_t*>(p);
  p += align256((size_t)n * 4);
  uint32_t* k_out = reinterpret_cast<uint32_t*>(p);
  p += align256((size_t)n * 4);
  uint64_t* v_in = reinterpret_cast<uint64_t*>(p);
  p += align256((size_t)n * 8);
  uint64_t* v_out = reinterpret_cast<uint64_t*>(p);
  p += align256((size_t)n * 8);
  int32_t* bounds = reinterpret_cast<int32_t*>(p);
  p += align256((size_t)nkeys * 8);
  size_t tmp_bytes = bwd_sort_temp_bytes(n, end_bit);
  void* tmp = p;

  // 1. per (token, side): dsigma, dx, one record per distinct table row
  const int64_t grid = (units + kWavesBwd / 2 - 1) / (kWavesBwd / 2);
  const size_t lds = score_bwd_lds_bytes(a.W > a.R ? a.W : a.R);
  auto k = bf16 ? sdm_score_bwd_kernel<true> : sdm_score_bwd_kernel<false>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k, dim3((unsigned)grid), dim3(kWavesBwd * 64), lds, stream, a, k_in, v_in);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // 2. records grouped by table row, slot order kept inside a row
  e = rocprim::radix_sort_pairs(tmp, tmp_bytes, k_in, k_out, v_in, v_out, (size_t)n, 0,
                                (unsigned)end_bit, stream);
  if (e != hipSuccess) return e;
  // 3. where each row's records start and end
  const int cgrid = (int)std::min<int64_t>((2 * nkeys + 255) / 256, 4096);
  hipLaunchKernelGGL(sdm_bwd_bounds_clear, dim3(cgrid), dim3(256), 0, stream, bounds, 2 * nkeys);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int bgrid = (int)std::min<int64_t>((n + 255) / 256, 65536);
  hipLaunchKernelGGL(sdm_bwd_bounds_kernel, dim3(bgrid), dim3(256), 0, stream, k_out, n,
                     (uint32_t)nkeys, bounds);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // 4. one wave per table row
  const unsigned rgrid = (unsigned)((nkeys + kRedWaves - 1) / kRedWaves);
  if (bf16)
    hipLaunchKernelGGL(sdm_score_bwd_reduce_kernel<true>, dim3(rgrid), dim3(kRedWaves * 64), 0,
                       stream, a, v_out, bounds);
  else
    hipLaunchKernelGGL(sdm_score_bwd_reduce_kernel<false>, dim3(rgrid), dim3(kRedWaves * 64), 0,
                       stream, a, v_out, bounds);
  return hipGetLastError();
}

}  // namespace sdm
