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
// row in LDS (per-row sums and each row's first event), then walks the distinct
// rows: it gathers each row once for dx and adds its dsigma*x into the table
// gradient with one float atomic per element.  The atomics make the sub-key
// gradient's summation order, and so its last bits, vary between runs; dq' and
// dk' are deterministic.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sdm_internal.h"

namespace sdm {

namespace {

constexpr int kWavesBwd = 4;  // waves per workgroup (2 tokens x 2 sides)

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

template <bool BF16>
__global__ void __launch_bounds__(kWavesBwd * 64) sdm_score_bwd_kernel(ScoreBwdArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int n_sub = a.n_sub;
  // per wave: row sums of dsigma for the two halves, then each row's first event
  float* acc = reinterpret_cast<float*>(smem) + (size_t)wave * 4 * n_sub;
  int32_t* first = reinterpret_cast<int32_t*>(acc + 2 * n_sub);

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
  float ds[2];
  int32_t ri[2], rj[2];
  float sw = 0.f;
#pragma unroll
  for (int u = 0; u < 2; u++) {
    const int r = u * 64 + lane;
    const bool on = r < k;
    const float w = on ? wt[r] : 0.f;
    ds[u] = on ? dw[r] : 0.f;
    sw += w * ds[u];
    const int32_t s = on ? idx[r] : 0;
    ri[u] = s / n_sub;
    rj[u] = s - ri[u] * n_sub;
    ds[u] = w;  // weight, turned into dsigma below
  }
  const float dot = wave_sum(sw);
#pragma unroll
  for (int u = 0; u < 2; u++) {
    const int r = u * 64 + lane;
    ds[u] = r < k ? ds[u] * (dw[r] - dot) : 0.f;
  }

  // ---- fold events that share a row --------------------------------------
  for (int i = lane; i < 2 * n_sub; i += 64) {
    acc[i] = 0.f;
    first[i] = 0x7fffffff;
  }
  wave_lds_sync();
#pragma unroll
  for (int u = 0; u < 2; u++) {
    const int r = u * 64 + lane;
    if (r < k) {
      atomicAdd(&acc[ri[u]], ds[u]);
      atomicAdd(&acc[n_sub + rj[u]], ds[u]);
      atomicMin(&first[ri[u]], r);
      atomicMin(&first[n_sub + rj[u]], r);
    }
  }
  wave_lds_sync();

  // ---- distinct rows: dx and the table gradient ---------------------------
  const int64_t xoff = unit * a.d_k;
  float* dsub_h = a.dsub + (int64_t)h * 2 * n_sub * dh;
  const int64_t cbase = (int64_t)h * 2 * n_sub * dh;
  for (int half = 0; half < 2; half++) {
    // x of this half and the running dx, dh <= 256: up to four elements a lane
    float xv[4], dxv[4];
#pragma unroll
    for (int c = 0; c < 4; c++) {
      const int e = c * 64 + lane;
      xv[c] = e < dh ? elem<BF16>(xin, xoff + half * dh + e) : 0.f;
      dxv[c] = 0.f;
    }
#pragma unroll
    for (int u = 0; u < 2; u++) {
      const int r = u * 64 + lane;
      const int row = half ? rj[u] : ri[u];
      const bool own = r < k && first[half * n_sub + row] == r;
      uint64_t bal = __ballot(own);
      while (bal) {  // wave-uniform walk over this chunk's distinct rows
        const int src = __builtin_ctzll(bal);
        bal &= bal - 1;
        const int rr = __shfl(row, src);
        const float g = acc[half * n_sub + rr];
        const int64_t crow = cbase + ((int64_t)half * n_sub + rr) * dh;
        float* drow = dsub_h + ((int64_t)half * n_sub + rr) * dh;
#pragma unroll
        for (int c = 0; c < 4; c++) {
          const int e = c * 64 + lane;
          if (e < dh) {
            dxv[c] += g * elem<BF16>(a.subkeys, crow + e);
            unsafeAtomicAdd(drow + e, g * xv[c]);
          }
        }
      }
    }
#pragma unroll
    for (int c = 0; c < 4; c++) {
      const int e = c * 64 + lane;
      if (e < dh) dx[half * dh + e] = dxv[c];
    }
  }
}

}  // namespace

size_t score_bwd_lds_bytes(int n_sub) { return (size_t)kWavesBwd * 4 * n_sub * sizeof(float); }

hipError_t launch_score_bwd(const ScoreBwdArgs& a, bool bf16, hipStream_t stream) {
  const int64_t units = (int64_t)a.S * a.T;
  if (units == 0) return hipSuccess;
  const int64_t grid = (units + kWavesBwd / 2 - 1) / (kWavesBwd / 2);
  const size_t lds = score_bwd_lds_bytes(a.n_sub);
  auto k = bf16 ? sdm_score_bwd_kernel<true> : sdm_score_bwd_kernel<false>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k, dim3((unsigned)grid), dim3(kWavesBwd * 64), lds, stream, a);
  return hipGetLastError();
}

}  // namespace sdm
