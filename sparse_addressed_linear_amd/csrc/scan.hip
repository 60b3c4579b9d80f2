// Sparse gated-delta scan over the explicit memory table, for gfx950.
//
// Method ("Sparse Delta Memory", gist.science summaries of paper 2607.07386;
// Spanish page "Mecanismo Central" items 1, 3, 4; French page "Mecanisme
// Central"): per (batch, head) stream and token t in order, the W selected
// write rows are decayed by alpha_t and moved toward v_t by beta_t * w (the
// gated delta update, written here as (1-c)*(alpha*M) + c*v with c = beta*w),
// every other row is untouched, and the output is the weighted sum of the R
// selected read rows taken after the write.
//
// GPU decomposition (all exact, because rows and columns evolve independently):
//   - stream          : one (b,h) table, N rows of d_v fp32.
//   - column slice    : CW = 4*LPR consecutive columns (>= 64 B per row access).
//   - slot partition  : rows with slot & (P-1) == p.  A token's events are split
//                       across the P partitions; each partition workgroup
//                       produces a partial read sum, added in partition order
//                       by sdm_partial_sum_kernel.
// One workgroup owns one (stream, slice, partition) and walks all tokens.
//
// Inside a workgroup, tokens are processed in blocks of NW tokens, one wave
// per token.  All row loads of a block are issued before any row of the block
// is stored, so every event sees the state before the block, unless the block
// itself wrote its slot earlier.  Such in-block dependences are found with an
// LDS hash of the block's write slots (slot -> bitmask of writing tokens):
//   write at token u of slot s : level = #{in-block writers of s before u}
//   read  at token u of slot s : level = #{in-block writers of s at or before u}
// Level-0 events use the speculative loads; level-L events reload after the
// level-(L-1) stores (barrier), and within a level all loads precede all stores
// (a level-L read of s must not see the level-L write of s by a later token).
// Writes of one slot get distinct levels, so a level never races with itself.
//
// gfx950 workgroup memory ordering: all waves of a workgroup share the CU's
// in-order vector L1, and __syncthreads() (workgroup-scope release/acquire)
// orders a wave's earlier global stores before another wave's later global
// loads, without draining the stores.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sdm_internal.h"

namespace sdm {

namespace {

constexpr int kEPL = 16;  // events per lane group kept in flight (registers)

__device__ __forceinline__ uint32_t mix32(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352dU;
  x ^= x >> 15;
  x *= 0x846ca68bU;
  x ^= x >> 16;
  return x;
}

__device__ __forceinline__ float4 load_v4(const void* v, bool bf16, int64_t off) {
  if (bf16) {
    const uint2 raw = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(v) + off);
    float4 r;
    r.x = __uint_as_float(raw.x << 16);
    r.y = __uint_as_float(raw.x & 0xffff0000u);
    r.z = __uint_as_float(raw.y << 16);
    r.w = __uint_as_float(raw.y & 0xffff0000u);
    return r;
  }
  return *reinterpret_cast<const float4*>(static_cast<const float*>(v) + off);
}

// Gated delta update of one float4 of a row: (1-c)*(a*m) + c*v, each operation
// rounded separately (no contraction), so c == 1 gives v and c == 0 gives a*m.
__device__ __forceinline__ float upd(float m, float a, float omc, float c, float v) {
#pragma clang fp contract(off)
  const float mt = a * m;
  const float keep = omc * mt;
  const float put = c * v;
  return keep + put;
}

// write strength c = beta*w and 1 - c, each rounded separately
__device__ __forceinline__ void gate(float beta, float w, float& c, float& omc) {
#pragma clang fp contract(off)
  c = beta * w;
  omc = 1.0f - c;
}

__device__ __forceinline__ float4 upd4(float4 m, float a, float omc, float c, float4 v) {
  return make_float4(upd(m.x, a, omc, c, v.x), upd(m.y, a, omc, c, v.y),
                     upd(m.z, a, omc, c, v.z), upd(m.w, a, omc, c, v.w));
}

__device__ __forceinline__ float4 fma4(float w, float4 x, float4 acc) {
  return make_float4(__fmaf_rn(w, x.x, acc.x), __fmaf_rn(w, x.y, acc.y),
                     __fmaf_rn(w, x.z, acc.z), __fmaf_rn(w, x.w, acc.w));
}

__device__ __forceinline__ float4 shfl_xor4(float4 a, int m) {
  return make_float4(__shfl_xor(a.x, m), __shfl_xor(a.y, m), __shfl_xor(a.z, m),
                     __shfl_xor(a.w, m));
}

__device__ __forceinline__ float4 add4(float4 a, float4 b) {
  return make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w);
}

}  // namespace

// LPR: lanes per row slice (CW = 4*LPR columns).  NW: waves = tokens per block.
template <int LPR, bool VBF16, int NW>
__global__ void __launch_bounds__(NW * 64, 1) sdm_scan_kernel(ScanArgs a) {
  constexpr int GPW = 64 / LPR;   // lane groups per wave
  constexpr int CAPW = GPW * kEPL;  // events per wave held in registers
  constexpr int CW = 4 * LPR;

  extern __shared__ __align__(16) unsigned char smem[];
  int32_t* hkey = reinterpret_cast<int32_t*>(smem);          // [2][hsize]
  uint32_t* hmask = reinterpret_cast<uint32_t*>(hkey + 2 * a.hsize);
  int32_t* lslot = reinterpret_cast<int32_t*>(hmask + 2 * a.hsize);  // [NW][lcap]
  float* lwt = reinterpret_cast<float*>(lslot + NW * a.lcap);
  int32_t* lmeta = reinterpret_cast<int32_t*>(lwt + NW * a.lcap);    // level | hpos<<8
  __shared__ int s_maxlvl[2];
  __shared__ int s_ovf[2];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int g = lane / LPR;  // lane group within the wave
  const int l = lane % LPR;  // float4 index within the row slice

  // workgroup -> (stream, column slice, partition); XCD-aware when possible so
  // that every workgroup of a stream shares one XCD's L2 for indices and v.
  const int Q = a.CS * a.P;
  int gi = blockIdx.x;
  if (a.xcd_map) {
    const int per = (a.S * Q) / 8;
    gi = (blockIdx.x % 8) * per + blockIdx.x / 8;
  }
  const int st = gi / Q;
  const int sub = gi % Q;
  const int cs = sub % a.CS;
  const int pp = sub / a.CS;
  const int c0 = cs * CW + 4 * l;  // this lane's first column
  const uint32_t pmask = (uint32_t)a.P - 1u;

  float* Mst = a.M + (int64_t)st * a.N * a.d_v + c0;
  const int hmsk = a.hsize - 1;

  int32_t* myslot = lslot + wave * a.lcap;
  float* mywt = lwt + wave * a.lcap;
  int32_t* mymeta = lmeta + wave * a.lcap;

  // initialise both hash tables and flags
  for (int i = tid; i < 2 * a.hsize; i += NW * 64) hkey[i] = -1, hmask[i] = 0u;
  if (tid < 2) s_maxlvl[tid] = 0, s_ovf[tid] = 0;
  __syncthreads();

  for (int t0 = 0, blk = 0; t0 < a.T; t0 += NW, blk++) {
    const int hb = blk & 1;
    int32_t* hk = hkey + hb * a.hsize;
    uint32_t* hm = hmask + hb * a.hsize;
    const int tok = t0 + wave;
    const bool valid = tok < a.T;
    const int64_t trow = (int64_t)st * a.T + tok;  // token row in [S][T]

    // ---- 1. compact this partition's events of the wave's token ----------
    int nw = 0, nr = 0;
    if (valid) {
      const int32_t* wi = a.widx + trow * a.W;
      const float* ww = a.wwt + trow * a.W;
      for (int c = 0; c < a.W; c += 64) {
        const int i = c + lane;
        int32_t s = -1;
        float w = 0.f;
        if (i < a.W) s = wi[i], w = ww[i];
        const bool f = s >= 0 && (((uint32_t)s & pmask) == (uint32_t)pp);
        const uint64_t bal = __ballot(f);
        if (f) {
          const int pos = nw + __popcll(bal & ((1ull << lane) - 1ull));
          myslot[pos] = s;
          mywt[pos] = w;
        }
        nw += __popcll(bal);
      }
      const int32_t* ri = a.ridx + trow * a.R;
      const float* rw = a.rwt + trow * a.R;
      for (int c = 0; c < a.R; c += 64) {
        const int i = c + lane;
        int32_t s = -1;
        float w = 0.f;
        if (i < a.R) s = ri[i], w = rw[i];
        const bool f = s >= 0 && (((uint32_t)s & pmask) == (uint32_t)pp);
        const uint64_t bal = __ballot(f);
        if (f) {
          const int pos = nw + nr + __popcll(bal & ((1ull << lane) - 1ull));
          myslot[pos] = s;
          mywt[pos] = w;
        }
        nr += __popcll(bal);
      }
    }
    const int ne = nw + nr;
    const bool fits = ne <= CAPW;
    wave_lds_sync();  // list entries written by other lanes are read below

    // ---- 2. speculative loads of every event row (state before the block) --
    float4 x[kEPL];
    if (fits) {
#pragma unroll
      for (int i = 0; i < kEPL; i++) {
        const int e = i * GPW + g;
        if (e < ne) x[i] = *reinterpret_cast<const float4*>(Mst + (int64_t)myslot[e] * a.d_v);
      }
    }

    // ---- 3. insert write slots into this block's hash ---------------------
    for (int e = lane; e < nw; e += 64) {
      const int32_t s = myslot[e];
      int h = (int)(mix32((uint32_t)s) & (uint32_t)hmsk);
      while (true) {
        const int32_t old = atomicCAS(&hk[h], -1, s);
        if (old == -1 || old == s) break;
        h = (h + 1) & hmsk;
      }
      atomicOr(&hm[h], 1u << wave);
      mymeta[e] = h << 8;
    }
    if (!fits && lane == 0) atomicOr(&s_ovf[hb], 1);
    // gates and this lane's slice of v for the wave's token
    float alpha = 0.f, beta = 0.f;
    float4 vv = make_float4(0.f, 0.f, 0.f, 0.f);
    if (valid) {
      alpha = a.alpha[trow];
      beta = a.beta[trow];
      vv = load_v4(a.v, VBF16, trow * a.d_v + c0);
    }
    __syncthreads();  // BAR1: all inserts visible; all speculative loads issued

    // the previous block's flags are no longer read by anyone: reset them
    if (tid == 0) s_maxlvl[hb ^ 1] = 0, s_ovf[hb ^ 1] = 0;

    // ---- 4. dependence levels ---------------------------------------------
    int mylvl = 0;
    const uint32_t wbefore = (1u << wave) - 1u;   // writers strictly before
    const uint32_t rbefore = (2u << wave) - 1u;   // writers at or before
    for (int e = lane; e < ne; e += 64) {
      const int32_t s = myslot[e];
      int h = (int)(mix32((uint32_t)s) & (uint32_t)hmsk);
      uint32_t m = 0u;
      while (true) {
        const int32_t k = hk[h];
        if (k == s) {
          m = hm[h];
          break;
        }
        if (k == -1) break;
        h = (h + 1) & hmsk;
      }
      const int lvl = __popc(m & (e < nw ? wbefore : rbefore));
      if (e < nw) mymeta[e] |= lvl;
      else mymeta[e] = lvl;
      mylvl = max(mylvl, lvl);
    }
    wave_lds_sync();  // levels written by other lanes are read below
    // wave max then workgroup max
    for (int o = 32; o > 0; o >>= 1) mylvl = max(mylvl, __shfl_xor(mylvl, o));
    if (lane == 0 && mylvl > 0) atomicMax(&s_maxlvl[hb], mylvl);
    const bool ovf = s_ovf[hb] != 0;  // set before BAR1

    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);

    if (!ovf) {
      // ---- 5. level-0 writes from the speculative loads -------------------
#pragma unroll
      for (int i = 0; i < kEPL; i++) {
        const int e = i * GPW + g;
        if (e < nw && (mymeta[e] & 0xff) == 0) {
          float c, omc;
          gate(beta, mywt[e], c, omc);
          *reinterpret_cast<float4*>(Mst + (int64_t)myslot[e] * a.d_v) =
              upd4(x[i], alpha, omc, c, vv);
        }
      }
      __syncthreads();  // BAR_A: level-0 stores before level-1 loads; max level known
      const int maxL = s_maxlvl[hb];
      for (int L = 1; L <= maxL; L++) {
#pragma unroll
        for (int i = 0; i < kEPL; i++) {
          const int e = i * GPW + g;
          if (e < ne && (mymeta[e] & 0xff) == L)
            x[i] = *reinterpret_cast<const float4*>(Mst + (int64_t)myslot[e] * a.d_v);
        }
        __syncthreads();  // every level-L load issued before any level-L store
#pragma unroll
        for (int i = 0; i < kEPL; i++) {
          const int e = i * GPW + g;
          if (e < nw && (mymeta[e] & 0xff) == L) {
            float c, omc;
            gate(beta, mywt[e], c, omc);
            *reinterpret_cast<float4*>(Mst + (int64_t)myslot[e] * a.d_v) =
                upd4(x[i], alpha, omc, c, vv);
          }
        }
        __syncthreads();  // level-L stores before level-(L+1) loads
      }
      // every read row now holds the value its token must see: sum them in
      // event order, so the result does not depend on where blocks start
#pragma unroll
      for (int i = 0; i < kEPL; i++) {
        const int e = i * GPW + g;
        if (e >= nw && e < ne) acc = fma4(mywt[e], x[i], acc);
      }
    } else {
      // ---- overflow path: some token has more events than fit in registers.
      // Per level: all reads (chunked, no stores), barrier, all writes
      // (chunked; writes of one level never share a slot), barrier.
      __syncthreads();  // max level known
      const int maxL = s_maxlvl[hb];
      for (int L = 0; L <= maxL; L++) {
        for (int base = nw; base < ne; base += CAPW) {
#pragma unroll
          for (int i = 0; i < kEPL; i++) {
            const int e = base + i * GPW + g;
            if (e < ne && (mymeta[e] & 0xff) == L)
              x[i] = *reinterpret_cast<const float4*>(Mst + (int64_t)myslot[e] * a.d_v);
          }
#pragma unroll
          for (int i = 0; i < kEPL; i++) {
            const int e = base + i * GPW + g;
            if (e < ne && (mymeta[e] & 0xff) == L) acc = fma4(mywt[e], x[i], acc);
          }
        }
        __syncthreads();  // level-L reads done before level-L writes store
        for (int base = 0; base < nw; base += CAPW) {
#pragma unroll
          for (int i = 0; i < kEPL; i++) {
            const int e = base + i * GPW + g;
            if (e < nw && (mymeta[e] & 0xff) == L)
              x[i] = *reinterpret_cast<const float4*>(Mst + (int64_t)myslot[e] * a.d_v);
          }
#pragma unroll
          for (int i = 0; i < kEPL; i++) {
            const int e = base + i * GPW + g;
            if (e < nw && (mymeta[e] & 0xff) == L) {
              float c, omc;
              gate(beta, mywt[e], c, omc);
              *reinterpret_cast<float4*>(Mst + (int64_t)myslot[e] * a.d_v) =
                  upd4(x[i], alpha, omc, c, vv);
            }
          }
        }
        __syncthreads();  // level-L stores before level-(L+1) loads
      }
    }

    // ---- 6. read sum across the wave's lane groups (fixed order) ----------
#pragma unroll
    for (int o = LPR; o < 64; o <<= 1) acc = add4(acc, shfl_xor4(acc, o));
    if (valid && g == 0) {
      float* dst = a.P == 1 ? a.out + trow * a.d_v + c0
                            : a.work + ((int64_t)pp * a.S * a.T + trow) * a.d_v + c0;
      *reinterpret_cast<float4*>(dst) = acc;
    }

    // ---- 7. clear this block's hash entries (all lookups are done) --------
    for (int e = lane; e < nw; e += 64) {
      const int h = mymeta[e] >> 8;
      hk[h] = -1;
      hm[h] = 0u;
    }
  }
}

// out[i] = sum over p of work[p][i], p ascending (deterministic).
__global__ void __launch_bounds__(256) sdm_partial_sum_kernel(const float* __restrict__ work,
                                                              float* __restrict__ out,
                                                              int64_t n4, int P) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) {
    float4 s = reinterpret_cast<const float4*>(work)[i];
    for (int p = 1; p < P; p++) s = add4(s, reinterpret_cast<const float4*>(work)[p * n4 + i]);
    reinterpret_cast<float4*>(out)[i] = s;
  }
}

// ----------------------------------------------------------------- launch --

template <int LPR, bool VBF16, int NW>
static hipError_t launch_scan_t(const ScanArgs& a, size_t lds, hipStream_t stream) {
  auto k = sdm_scan_kernel<LPR, VBF16, NW>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k, dim3(a.S * a.CS * a.P), dim3(NW * 64), lds, stream, a);
  return hipGetLastError();
}

ScanPlan plan_scan(int S, int T, int64_t N, int d_v, int W, int R) {
  ScanPlan p{};
  p.lpr = (d_v % 32 == 0) ? 8 : 4;
  p.CS = d_v / (4 * p.lpr);
  p.nw = 8;
  // partitions: enough workgroups to occupy every CU, while keeping enough
  // events per token and partition to fill a wave.
  int P = 1;
  while (P < 64 && (int64_t)S * p.CS * (P * 2) <= kTargetWorkgroups &&
         (W + R) / (P * 2) >= 16 && P * 2 <= N)
    P *= 2;
  p.P = P;
  int64_t hs = 1;
  while (hs < 2LL * p.nw * W) hs *= 2;
  p.hsize = (int)hs;
  p.lcap = W + R;
  p.lds = (size_t)2 * p.hsize * 8 + (size_t)p.nw * p.lcap * 12;
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
  hipError_t e;
#define SDM_SCAN_CASE(LPR_, NW_)                                                 \
  if (p.lpr == LPR_ && p.nw == NW_) {                                            \
    e = vbf16 ? launch_scan_t<LPR_, true, NW_>(a, p.lds, stream)                 \
              : launch_scan_t<LPR_, false, NW_>(a, p.lds, stream);               \
  } else
  SDM_SCAN_CASE(8, 8)
  SDM_SCAN_CASE(4, 8) { return hipErrorInvalidValue; }
#undef SDM_SCAN_CASE
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
