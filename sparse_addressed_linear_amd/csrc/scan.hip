// Sparse gated-delta scan over the explicit memory table, for gfx950: the
// launch planner, the plain-load build of the kernel (scan_kernel.h) and the
// deterministic sum of the partitions' partial reads.
#include "scan_kernel.h"

namespace sdm {

// out[i] = sum over p of work[p][i], p ascending (deterministic); the
// partials are read once, as streaming loads.
__global__ void __launch_bounds__(256) sdm_partial_sum_kernel(const float* __restrict__ work,
                                                              float* __restrict__ out,
                                                              int64_t n4, int P) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) {
    const float* w0 = work + 4 * i;
    float4 s = make_float4(__builtin_nontemporal_load(w0), __builtin_nontemporal_load(w0 + 1),
                           __builtin_nontemporal_load(w0 + 2), __builtin_nontemporal_load(w0 + 3));
    for (int p = 1; p < P; p++) {
      const float* wp = work + 4 * (p * n4 + i);
      s = add4(s, make_float4(__builtin_nontemporal_load(wp), __builtin_nontemporal_load(wp + 1),
                              __builtin_nontemporal_load(wp + 2), __builtin_nontemporal_load(wp + 3)));
    }
    reinterpret_cast<float4*>(out)[i] = s;
  }
}

ScanPlan plan_scan(int S, int T, int64_t N, int d_v, int W, int R, bool tape) {
  ScanPlan p{};
  // partitions for cs column slices: enough workgroups to occupy every CU,
  // while keeping enough events per token and partition to fill a wave
  auto parts = [&](int cs) {
    int P = 1;
    while (P < 64 && (int64_t)S * cs * (P * 2) <= kTargetWorkgroups &&
           (W + R) / (P * 2) >= 8 && P * 2 <= N)
      P *= 2;
    return P;
  };
  // registers per lane group for P partitions and lanes-per-slice lpr: the
  // mean events of a token in one partition plus three standard deviations
  // (partitions are hashed, so the count is close to binomial); rarer tokens
  // take the overflow path, which costs little at that rate, while every
  // register slot past a token's events is a padding load
  auto epl_for = [&](int P, int lpr) {
    const double mean = (double)(W + R) / P;
    const double need = mean + 3.0 * sqrt(mean * (1.0 - 1.0 / P));
    const int gpw = 64 / lpr;
    return need <= 8 * gpw ? 8 : (need <= 12 * gpw ? 12 : (need <= 16 * gpw ? 16 : 0));
  };
  // row slices: 128 B (64 B where d_v is not a multiple of 32), or 256 B
  // where d_v allows and they still fill the GPU with few partitions, at most
  // (2W+R)/24, so that the partial read sums add at most about 8% to the
  // scan's bytes, and a token's events of a partition still fit a wave's
  // registers.  Wider slices mean fewer workgroups repeat a token's index work
  // and fewer, larger row accesses per workgroup.  Measured (same box): Large
  // 2.86 ms with 256 B slices against 3.14 with 128 B; Long 50.3 ms against
  // 55.9 with 128 B and 52.9 with whole 512 B rows (16 partitions, half the
  // register slots padding)
  p.lpr = d_v % 32 == 0 ? 8 : 4;
  if (d_v % 64 == 0) {
    const int cs = d_v / 64;
    const int pw = parts(cs);
    if ((int64_t)S * cs * pw >= kTargetWorkgroups && pw * 24 <= 2 * W + R &&
        epl_for(pw, 16) != 0)
      p.lpr = 16;
  }
  p.CS = d_v / (4 * p.lpr);
  p.P = parts(p.CS);
  const int P = p.P;
  // one token per stream (decoding): one-wave workgroups, so that several
  // share a CU and the launch runs in one round instead of idling 7 waves each
  p.nw = (T == 1 && !tape) ? 1 : 8;
  p.epl = epl_for(P, p.lpr);
  if (p.epl == 0) p.epl = 16;  // most tokens take the overflow path
  int64_t hs = 1;
  while (hs < 2LL * p.nw * W) hs *= 2;
  p.hsize = (int)hs;
  p.lcap = W + R;
  p.lds = (size_t)p.hsize * 8 + (size_t)p.nw * p.lcap * 12;
  p.work_bytes = P > 1 ? (size_t)P * S * T * d_v * sizeof(float) : 0;
  return p;
}

hipError_t launch_scan(const ScanArgs& a0, const ScanPlan& p, bool vbf16, hipStream_t stream) {
  ScanArgs a = a0;
  a.CS = p.CS;
  a.P = p.P;
  a.hsize = p.hsize;
  a.lcap = p.lcap;
  a.xcd_map = ((int64_t)a.S * a.CS * a.P) % 8 == 0 ? 1 : 0;
  if (a.T == 0) return hipSuccess;
  const bool buf = a.N * a.d_v * 4 <= kBufMaxBytes;
  hipError_t e = buf ? launch_scan_kernel_buf(a, p, vbf16, stream)
                     : launch_scan_kernel<false>(a, p, vbf16, stream);
  if (e != hipSuccess) return e;
  if (p.P > 1) {
    const int64_t n4 = (int64_t)a.S * a.T * a.d_v / 4;
    int grid = (int)((n4 + 255) / 256);
    if (grid > 4096) grid = 4096;
    hipLaunchKernelGGL(sdm_partial_sum_kernel, dim3(grid), dim3(256), 0, stream, a.work, a.out,
                       n4, p.P);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace sdm
