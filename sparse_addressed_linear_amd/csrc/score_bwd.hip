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
// event), lists the distinct rows in the order of their first events, and
// walks them eight at a time: it gathers each row once for dx and adds its
// dsigma*x into the table gradient with one float atomic per element.  The
// atomics make the sub-key gradient's summation order, and so its last bits,
// vary between runs; dq' and dk' are summed in rank order.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sdm_internal.h"

namespace sdm {

namespace {

constexpr int kWavesBwd = 8;  // waves per workgroup (4 tokens x 2 sides)

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
__global__ void __launch_bounds__(kWavesBwd * 64) sdm_score_bwd_kernel(ScoreBwdArgs a) {
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
  const void* xin = side ? a.qp : a.kp;
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
  const int64_t xoff = unit * a.d_k;
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
    float xv[4], dxv[4];
#pragma unroll
    for (int c = 0; c < 4; c++) {
      const int e = c * 64 + lane;
      xv[c] = e < dh ? elem<BF16>(xin, xoff + half * dh + e) : 0.f;
      dxv[c] = 0.f;
    }
    const int64_t hbase = cbase + (int64_t)half * n_sub * dh;
    for (int b0 = 0; b0 < nd; b0 += 8) {
      // eight rows' elements in flight, then the sums and the atomics
      float cv[8][4];
#pragma unroll
      for (int j = 0; j < 8; j++) {
        const int32_t row = b0 + j < nd ? dist[b0 + j].key : 0;
#pragma unroll
        for (int c = 0; c < 4; c++) {
          const int e = c * 64 + lane;
          cv[j][c] = e < dh ? elem<BF16>(a.subkeys, hbase + (int64_t)row * dh + e) : 0.f;
        }
      }
#pragma unroll
      for (int j = 0; j < 8; j++) {
        if (b0 + j < nd) {
          const float g = dist[b0 + j].sum;
          float* drow = a.dsub + hbase + (int64_t)dist[b0 + j].key * dh;
#pragma unroll
          for (int c = 0; c < 4; c++) {
            const int e = c * 64 + lane;
            if (e < dh) {
              dxv[c] += g * cv[j][c];
              unsafeAtomicAdd(drow + e, g * xv[c]);
            }
          }
        }
      }
    }
#pragma unroll
    for (int c = 0; c < 4; c++) {
      const int e = c * 64 + lane;
      if (e < dh) dx[half * dh + e] = dxv[c];
    }
    wave_lds_sync();  // the distinct list is rebuilt for the next half
  }
}

}  // namespace

size_t score_bwd_lds_bytes(int kmax) {
  return (size_t)kWavesBwd * (2 * row_table_size(kmax) + kmax) * sizeof(RowEnt);
}

hipError_t launch_score_bwd(const ScoreBwdArgs& a, bool bf16, hipStream_t stream) {
  const int64_t units = (int64_t)a.S * a.T;
  if (units == 0) return hipSuccess;
  const int64_t grid = (units + kWavesBwd / 2 - 1) / (kWavesBwd / 2);
  const size_t lds = score_bwd_lds_bytes(a.W > a.R ? a.W : a.R);
  auto k = bf16 ? sdm_score_bwd_kernel<true> : sdm_score_bwd_kernel<false>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k, dim3((unsigned)grid), dim3(kWavesBwd * 64), lds, stream, a);
  return hipGetLastError();
}

}  // namespace sdm
