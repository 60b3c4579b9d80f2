// Product-key addressing for Sparse Delta Memory: launch selection.  The
// kernel and its design notes are in score_topk_impl.h; its instances are
// compiled in score_topk_t{1,2,4,8}.hip.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "score_topk_impl.h"

namespace sdm {

extern template hipError_t launch_score_t<1>(const ScoreArgs&, bool, int, hipStream_t);
extern template hipError_t launch_score_t<2>(const ScoreArgs&, bool, int, hipStream_t);
extern template hipError_t launch_score_t<4>(const ScoreArgs&, bool, int, hipStream_t);
extern template hipError_t launch_score_t<8>(const ScoreArgs&, bool, int, hipStream_t);

// Sub-key tables in the order the MFMA A operand takes them: for head h, half
// c, tile t (sub-keys 16t .. 16t+15) and K step ks < score_ksteps(dh)
// (elements 32ks .. 32ks+31),
// 64 pieces of 8 bf16, piece l = sub-key 16t + l%16, elements
// 32ks + 8*(l/16) .. +8 (zero past dh).  One thread per 16-byte piece.
__global__ void __launch_bounds__(256) sdm_pack_subkeys_kernel(const uint16_t* __restrict__ C,
                                                              uint4* __restrict__ packed,
                                                              int64_t pieces, int n_sub, int dh,
                                                              int ksteps) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= pieces) return;
  const int l = (int)(i & 63);
  int64_t r = i >> 6;
  const int ks = (int)(r % ksteps);
  r /= ksteps;
  const int n_tiles = n_sub / 16;
  const int t = (int)(r % n_tiles);
  const int64_t hc = r / n_tiles;  // head * 2 + half
  const int d0 = 32 * ks + 8 * (l >> 4);
  uint4 v = make_uint4(0u, 0u, 0u, 0u);
  if (d0 < dh)
    v = *reinterpret_cast<const uint4*>(C + (hc * n_sub + 16 * t + (l & 15)) * dh + d0);
  packed[i] = v;
}

size_t score_topk_workspace_bytes(int H, int n_sub, int d_k, bool bf16) {
  if (!bf16) return 0;
  return (size_t)H * 2 * (n_sub / 16) * score_ksteps(d_k / 2) * 1024;
}

size_t score_topk_lds_bytes(int n_sub, int W, int R) {
  (void)n_sub;
  return score_smem(W, R).total;
}

hipError_t launch_pack_subkeys(const ScoreArgs& a, hipStream_t stream) {
  if (a.packed == nullptr) return hipErrorInvalidValue;  // the packed fragments' home
  const int dh = a.d_k / 2;
  const int ksteps = score_ksteps(dh);
  const int64_t pieces = (int64_t)a.H * 2 * (a.n_sub / 16) * ksteps * 64;
  hipLaunchKernelGGL(sdm_pack_subkeys_kernel, dim3((unsigned)((pieces + 255) / 256)), dim3(256), 0,
                     stream, static_cast<const uint16_t*>(a.subkeys),
                     static_cast<uint4*>(a.packed), pieces, a.n_sub, dh, ksteps);
  return hipGetLastError();
}

hipError_t launch_score_topk(const ScoreArgs& a, bool bf16, bool pack, hipStream_t stream) {
  if (a.T == 0) return hipSuccess;
  if (bf16 && a.packed == nullptr) return hipErrorInvalidValue;  // the packed fragments' home
  if (bf16 && pack) {
    const hipError_t e = launch_pack_subkeys(a, stream);
    if (e != hipSuccess) return e;
  }
  const int tiles = (a.n_sub + 15) / 16;
  const int nt = (tiles + kWaves - 1) / kWaves;  // sub-key tiles per wave
  const int g = pruned_grid_size(a.W > a.R ? a.W : a.R);
  const int npl2 = (g + 63) / 64;
  if (npl2 > kGridMax / 64) return hipErrorInvalidValue;
  if (nt <= 1) return launch_score_t<1>(a, bf16, npl2, stream);
  if (nt <= 2) return launch_score_t<2>(a, bf16, npl2, stream);
  if (nt <= 4) return launch_score_t<4>(a, bf16, npl2, stream);
  if (nt <= 8) return launch_score_t<8>(a, bf16, npl2, stream);
  return hipErrorInvalidValue;
}

}  // namespace sdm
