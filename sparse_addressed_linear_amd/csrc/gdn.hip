// Dense gated-delta recurrence (the gated DeltaNet state that Sparse Delta
// Memory extends; Spanish page "Planteamiento del Problema" / "Metodologia"),
// the IsoFLOP baseline of the sparse path, for gfx950:
//   S_t = alpha_t S_{t-1} + beta_t (v_t - alpha_t S_{t-1} k_t) k_t^T
//   o_t = S_t q_t
// One workgroup per (b,h) stream keeps S (d_v x d_k = 128 x 128 fp32) in
// registers: 512 threads, each a 4-row x 8-column tile.  Per token, with
// p = S k and r = S q taken from the old state:
//   e = beta (v - alpha p),  o = alpha r + e (k . q),  S <- alpha S + e k^T
// (o = S_t q expanded with S_t = alpha S + e k^T).  The registers hold S as
// A * Shat with a scalar A (the product of the alphas since the last fold), so
// the decay costs one multiply per token instead of one per element:
//   A' = alpha A,  Shat <- Shat + (e / A') k^T  (one FMA per element),
// and A is folded back into Shat at every chunk of tokens (and at once when
// alpha A falls below 2^-30, alpha = 0 included).  The two row reductions
// over the 16 column tiles of a row run as one reduce-scatter butterfly; all
// cross-lane moves stay inside 16-lane DPP rows (no LDS round trips).
// Bound: fp32 VALU (4 d_v d_k FMA per token), not HBM.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sdm_internal.h"

namespace sdm {

namespace {

constexpr int kD = 128;         // d_k = d_v
constexpr int kThr = 512;       // threads per stream
constexpr int kTC = 16;         // tokens staged per chunk
constexpr int kChunkF4 = kTC * (3 * kD + 4) / 4;  // float4 per chunk (k, q, v, gates)

__device__ __forceinline__ float4 ld4(const float* p) { return *reinterpret_cast<const float4*>(p); }

// v of lane n of this lane's row of 16 (DPP row broadcast)
template <int N>
__device__ __forceinline__ float row_bcast(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x150 + N, 0xF, 0xF, false));
}

}  // namespace

template <bool BF16>
__device__ __forceinline__ float4 load_in4(const void* base, int64_t off) {
  if (BF16) {
    const uint2 raw = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(base) + off);
    return make_float4(__uint_as_float(raw.x << 16), __uint_as_float(raw.x & 0xffff0000u),
                       __uint_as_float(raw.y << 16), __uint_as_float(raw.y & 0xffff0000u));
  }
  return ld4(static_cast<const float*>(base) + off);
}

// Staged chunk layout in LDS (floats): k[kTC][128] | q[kTC][128] | v[kTC][128] | ab[kTC][4]
template <bool BF16>
__device__ __forceinline__ float4 chunk_elem(const GdnArgs& a, int st, int tc0, int f4) {
  // f4 indexes float4 slots of the chunk layout above
  const int per = kD / 4;  // float4 per vector
  int seg = f4 / (kTC * per);
  float4 r = make_float4(0.f, 0.f, 0.f, 0.f);
  if (seg < 3) {
    const int rem = f4 - seg * kTC * per;
    const int t = tc0 + rem / per;
    const int c = (rem % per) * 4;
    if (t < a.T) {
      const int64_t row = (int64_t)st * a.T + t;
      const void* src = seg == 0 ? a.k : (seg == 1 ? a.q : a.v);
      r = load_in4<BF16>(src, row * kD + c);
    }
  } else {
    const int t = tc0 + (f4 - 3 * kTC * per);
    if (t < a.T) {
      const int64_t row = (int64_t)st * a.T + t;
      r.x = a.alpha[row];
      r.y = a.beta[row];
    }
  }
  return r;
}

template <bool BF16>
__global__ void __launch_bounds__(kThr, 1) sdm_gdn_kernel(GdnArgs a) {
  __shared__ __align__(16) float stage[2][kChunkF4 * 4];
  const int tid = threadIdx.x;
  const int st = blockIdx.x;
  const int cg = tid & 15;        // column tile: columns 8cg .. 8cg+7
  const int rg = tid >> 4;        // row tile: rows 4rg .. 4rg+3
  const int b0 = cg & 1, b1 = (cg >> 1) & 1, b2 = (cg >> 2) & 1, b3 = (cg >> 3) & 1;
  const int lane = tid & 63;

  float* Sg = a.S + (int64_t)st * kD * kD;
  float s[4][8];
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const float4 x0 = ld4(Sg + (4 * rg + i) * kD + 8 * cg);
    const float4 x1 = ld4(Sg + (4 * rg + i) * kD + 8 * cg + 4);
    s[i][0] = x0.x; s[i][1] = x0.y; s[i][2] = x0.z; s[i][3] = x0.w;
    s[i][4] = x1.x; s[i][5] = x1.y; s[i][6] = x1.z; s[i][7] = x1.w;
  }

  constexpr int F4PT = (kChunkF4 + kThr - 1) / kThr;  // float4 per thread per chunk
  float4 pre[F4PT];
  // stage chunk 0
#pragma unroll
  for (int u = 0; u < F4PT; u++) {
    const int f4 = tid + u * kThr;
    if (f4 < kChunkF4) reinterpret_cast<float4*>(stage[0])[f4] = chunk_elem<BF16>(a, st, 0, f4);
  }
  __syncthreads();

  float A = 1.0f;  // S = A * s
  for (int tc0 = 0, cb = 0; tc0 < a.T; tc0 += kTC, cb ^= 1) {
    // prefetch the next chunk into registers
    const bool more = tc0 + kTC < a.T;
    if (more) {
#pragma unroll
      for (int u = 0; u < F4PT; u++) {
        const int f4 = tid + u * kThr;
        if (f4 < kChunkF4) pre[u] = chunk_elem<BF16>(a, st, tc0 + kTC, f4);
      }
    }
    const float* K = stage[cb];
    const float* Q = K + kTC * kD;
    const float* V = Q + kTC * kD;
    const float* AB = V + kTC * kD;
    const int nt = min(kTC, a.T - tc0);
    // k . q of each of the chunk's tokens, computed once (32 threads a token)
    // into the third slot of its gates instead of by every thread per token
    {
      const int tt = tid >> 5, sub = tid & 31;
      float d = 0.f;
      if (tt < nt) {
        const float4 kx = ld4(K + tt * kD + 4 * sub), qx = ld4(Q + tt * kD + 4 * sub);
        d = fmaf(kx.x, qx.x, d);
        d = fmaf(kx.y, qx.y, d);
        d = fmaf(kx.z, qx.z, d);
        d = fmaf(kx.w, qx.w, d);
      }
#pragma unroll
      for (int o = 1; o < 32; o <<= 1) d += xor_shuffle(d, o, lane);
      if (sub == 0 && tt < nt) stage[cb][3 * kTC * kD + tt * 4 + 2] = d;
    }
    __syncthreads();
    for (int tt = 0; tt < nt; tt++) {
      const float4 k0 = ld4(K + tt * kD + 8 * cg), k1 = ld4(K + tt * kD + 8 * cg + 4);
      const float4 q0 = ld4(Q + tt * kD + 8 * cg), q1 = ld4(Q + tt * kD + 8 * cg + 4);
      const float kk[8] = {k0.x, k0.y, k0.z, k0.w, k1.x, k1.y, k1.z, k1.w};
      const float qq[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
      const float alpha = AB[tt * 4 + 0], beta = AB[tt * 4 + 1];
      // partial p (values 0..3) and r (values 4..7) of this tile's rows
      float val[8];
#pragma unroll
      for (int i = 0; i < 4; i++) {
        float p = 0.f, r = 0.f;
#pragma unroll
        for (int j = 0; j < 8; j++) {
          p = fmaf(s[i][j], kk[j], p);
          r = fmaf(s[i][j], qq[j], r);
        }
        val[i] = p;
        val[4 + i] = r;
      }
      const float kq = AB[tt * 4 + 2];
      // reduce-scatter over the 16 column tiles: lane keeps value 4b3+2b2+b1
      float h4[4];
#pragma unroll
      for (int u = 0; u < 4; u++) {
        const float send = b3 ? val[u] : val[4 + u];
        const float keep = b3 ? val[4 + u] : val[u];
        h4[u] = keep + xor_shuffle(send, 8, lane);
      }
      float h2[2];
#pragma unroll
      for (int u = 0; u < 2; u++) {
        const float send = b2 ? h4[u] : h4[2 + u];
        const float keep = b2 ? h4[2 + u] : h4[u];
        h2[u] = keep + xor_shuffle(send, 4, lane);
      }
      float h1;
      {
        const float send = b1 ? h2[0] : h2[1];
        const float keep = b1 ? h2[1] : h2[0];
        h1 = keep + xor_shuffle(send, 2, lane);
      }
      h1 += xor_shuffle(h1, 1, lane);
      // lane holds row ri = 2b2+b1 of the tile: p if b3 == 0, r if b3 == 1
      // (h1 is of the scaled state: the true p or r is A * h1)
      const int ri = 2 * b2 + b1;
      const float vrow = V[tt * kD + 4 * rg + ri];
      const float aA = alpha * A;                         // A' (uniform)
      const float e_own = beta * (vrow - aA * h1);        // meaningful where b3 == 0
      const float e_row = xor_shuffle(e_own, 8, lane);   // e of the row, at b3 == 1
      if (b3 == 1 && b0 == 0 && tc0 + tt < a.T) {
        const float o = fmaf(aA, h1, e_row * kq);
        a.out[((int64_t)st * a.T + tc0 + tt) * kD + 4 * rg + ri] = o;
      }
      float inv;
      if (aA < 0x1p-30f) {  // fold now: s <- A' s, A <- 1 (alpha = 0 clears s)
#pragma unroll
        for (int i = 0; i < 4; i++)
#pragma unroll
          for (int j = 0; j < 8; j++) s[i][j] *= aA;
        A = 1.0f;
        inv = 1.0f;
      } else {
        A = aA;
        inv = __builtin_amdgcn_rcpf(aA);  // hardware reciprocal (1 ulp)
      }
      // e / A' of the tile's 4 rows (held at lanes b3=0, 2b2+b1 = i)
      const float es = e_own * inv;
      const float e[4] = {row_bcast<0>(es), row_bcast<2>(es), row_bcast<4>(es), row_bcast<6>(es)};
#pragma unroll
      for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 8; j++) s[i][j] = fmaf(e[i], kk[j], s[i][j]);
    }
    // fold A into s once per chunk
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
      for (int j = 0; j < 8; j++) s[i][j] *= A;
    A = 1.0f;
    if (more) {
      // everyone is done reading stage[cb ^ 1] (used two chunks ago)
#pragma unroll
      for (int u = 0; u < F4PT; u++) {
        const int f4 = tid + u * kThr;
        if (f4 < kChunkF4) reinterpret_cast<float4*>(stage[cb ^ 1])[f4] = pre[u];
      }
    }
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < 4; i++) {
    float* dst = Sg + (4 * rg + i) * kD + 8 * cg;
    *reinterpret_cast<float4*>(dst) = make_float4(s[i][0], s[i][1], s[i][2], s[i][3]);
    *reinterpret_cast<float4*>(dst + 4) = make_float4(s[i][4], s[i][5], s[i][6], s[i][7]);
  }
}

hipError_t launch_gdn(const GdnArgs& a, bool bf16, hipStream_t stream) {
  if (a.nS == 0) return hipSuccess;
  if (bf16) hipLaunchKernelGGL(sdm_gdn_kernel<true>, dim3(a.nS), dim3(kThr), 0, stream, a);
  else hipLaunchKernelGGL(sdm_gdn_kernel<false>, dim3(a.nS), dim3(kThr), 0, stream, a);
  return hipGetLastError();
}

}  // namespace sdm
