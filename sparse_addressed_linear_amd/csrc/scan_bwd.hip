// Reverse sweep of the sparse gated-delta scan: gradients of the write/read
// recurrence, for gfx950.
//
// The forward ("Sparse Delta Memory", gist.science summaries of paper
// 2607.07386; Spanish page "Mecanismo Central" items 3 and 4) is, per stream
// and token t: for each write slot s_r with weight w_r, c = beta*w_r and
// M_t[s_r] = (1-c)*(alpha*M_{t-1}[s_r]) + c*v_t; then o_t = sum_r r_r*M_t[ridx_r].
// M0 is a learned parameter (Spanish page "Estado Inicial Aprendido"), so the
// sweep also returns dL/dM0.  Adjoint of token t, taken in reverse time order
// (the read, then the write), with dM holding dL/dM_t:
//   read  r: dr_r = <dO_t, M_t[ridx_r]>;  dM[ridx_r] += r_r*dO_t
//   write r: G = dM[s_r], old = M_{t-1}[s_r] (the forward's tape);
//            dc = <G, v_t - alpha*old>;  dw_r = beta*dc;  dbeta_t += w_r*dc;
//            dalpha_t += (1-c)*<G, old>;  dv_t += c*G;
//            dM[s_r] = (1-c)*alpha*G;  M[s_r] = old (the table walks back to M0).
//
// GPU decomposition: one workgroup per (stream, slot partition), whole rows
// (LPR = d_v/4 lanes per row, GPW = 64/LPR rows per wave instruction), so the
// per-event dot products finish inside the workgroup.  A token's per-token sums
// (dv, dalpha, dbeta) are partial per partition and added in partition order
// by sdm_bwd_sum_kernel (deterministic).
//
// Tokens go in blocks of NW = 8, one wave per token, latest token in wave 0.
// Processing order inside a block: wave 0's reads, wave 0's writes, wave 1's
// reads, ...  Every event reads and writes state (dM always, M for writes), so
// an event's level is the number of block events on its slot that come before
// it in that order (LDS hash: slot -> bit 2*wave + kind).  Events of one level
// touch distinct slots, so a level has no internal hazard; a barrier separates
// level L's stores from level L+1's loads.  Level-0 rows are loaded for every
// event up front; level-L events reload theirs.  A token with more events in
// its partition than a wave holds in registers sends its block down a serial
// path (one wave at a time, in processing order, in register-sized chunks).
// So does a token that reads one slot more than once (allowed: only write
// slots must be distinct): its reads share a hash bit and would share a level,
// so the serial path takes that block's reads one at a time, each adding its
// own share to the row's gradient.
//
// Memory ordering is the forward kernel's: waves of a workgroup share the CU's
// in-order vector L1, and a workgroup barrier orders earlier global stores
// before later global loads of other waves.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "scan_common.h"
#include "sdm_internal.h"

namespace sdm {

using namespace scanc;

namespace {

constexpr int kNW = 8;          // waves (tokens) per block
constexpr int kLvl = 0x7f;      // meta: level bits
constexpr int kWrite = 0x80;    // meta: write event (else read)

__device__ __forceinline__ float dot4(float4 a, float4 b) {
  return a.x * b.x + a.y * b.y + a.z * b.z + a.w * b.w;
}

__device__ __forceinline__ float4 scale4(float s, float4 a) {
  return make_float4(s * a.x, s * a.y, s * a.z, s * a.w);
}

// sum over the LPR lanes of a lane group (every lane of the wave active)
template <int LPR>
__device__ __forceinline__ float group_sum(float x) {
#pragma unroll
  for (int o = 1; o < LPR; o <<= 1) x += __shfl_xor(x, o);
  return x;
}

// MC: 64-wide chunks of a token's index lists (W, R <= 64*MC).
template <int LPR, bool VBF16, int EPL, int MC>
__global__ void __launch_bounds__(kNW * 64, 1) sdm_scan_bwd_kernel(ScanBwdArgs a) {
  constexpr int GPW = 64 / LPR;    // rows per wave instruction
  constexpr int CAPW = GPW * EPL;  // events per wave held in registers
  constexpr int NT = kNW * 64;

  extern __shared__ __align__(16) unsigned char smem[];
  uint64_t* htab = reinterpret_cast<uint64_t*>(smem);              // [hsize]
  int32_t* lslot = reinterpret_cast<int32_t*>(htab + a.hsize);     // [NW][lcap]
  float* lwt = reinterpret_cast<float*>(lslot + kNW * a.lcap);     // [NW][lcap]
  int32_t* lmeta = reinterpret_cast<int32_t*>(lwt + kNW * a.lcap);  // [NW][lcap]
  __shared__ int s_maxl, s_ovf;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int g = lane / LPR;  // lane group: one row
  const int l = lane % LPR;  // float4 within the row

  int gi = blockIdx.x;
  if (a.xcd_map) {
    const int per = (a.S * a.P) / 8;
    gi = (blockIdx.x % 8) * per + blockIdx.x / 8;
  }
  const int st = gi / a.P;
  const int pp = gi % a.P;
  const uint32_t pmask = (uint32_t)a.P - 1u;
  const int c0 = 4 * l;
  const int hmsk = a.hsize - 1;
  const int64_t sbase = (int64_t)st * a.N * a.d_v + c0;
  float* Mst = a.M + sbase;
  float* dMst = a.dM + sbase;
  int32_t* sl = lslot + wave * a.lcap;
  float* wl = lwt + wave * a.lcap;
  int32_t* ml = lmeta + wave * a.lcap;
  // an event whose slot lies outside [0, N) belongs to no partition (the
  // forward scan ignored it); partition 0 gives its weight a zero gradient
  const uint32_t nlim = (uint32_t)a.N;
  auto in_part = [&](int32_t s) {
    return (uint32_t)s < nlim && ((mix32((uint32_t)s) >> 16) & pmask) == (uint32_t)pp;
  };
  const uint64_t below = (1ull << lane) - 1ull;

  for (int i = tid; i < a.hsize; i += NT) htab[i] = kEmpty;
  __syncthreads();
  const int nblk = (a.T + kNW - 1) / kNW;

  // ---- the next block's index lists, weights, gates, v and dO, one block
  // ahead in registers (unconditional loads at clamped addresses) ----------
  int32_t ps[MC], qs[MC];
  float pw[MC], qw[MC];
  float nal, nbe;
  float4 nv, ndO;
  auto prefetch = [&](int blk) {
    const int tk = blk * kNW + (kNW - 1 - wave);
    const bool ok = blk >= 0 && tk < a.T;
    const int64_t tr = (int64_t)st * a.T + (ok ? tk : 0);
#pragma unroll
    for (int c = 0; c < MC; c++) {
      if (c * 64 < a.W) {
        const int i = c * 64 + lane < a.W ? c * 64 + lane : a.W - 1;
        ps[c] = a.widx[tr * a.W + i];
        pw[c] = a.wwt[tr * a.W + i];
      }
      if (c * 64 < a.R) {
        const int i = c * 64 + lane < a.R ? c * 64 + lane : a.R - 1;
        qs[c] = a.ridx[tr * a.R + i];
        qw[c] = a.rwt[tr * a.R + i];
      }
    }
    nal = a.alpha[tr];
    nbe = a.beta[tr];
    nv = load_v4(a.v, VBF16, tr * a.d_v + c0);
    ndO = *reinterpret_cast<const float4*>(a.dout + tr * a.d_v + c0);
  };
  prefetch(nblk - 1);

  for (int b = nblk - 1; b >= 0; b--) {
    const int tok = b * kNW + (kNW - 1 - wave);  // wave 0: the block's latest token
    const bool valid = tok < a.T;
    const int64_t trow = (int64_t)st * a.T + (valid ? tok : 0);
    if (tid == 0) s_maxl = 0, s_ovf = 0;

    // ---- 1. this token's events of the partition: reads, then writes ------
    int nr = 0, nwr = 0;
    if (valid) {
#pragma unroll
      for (int c = 0; c < MC; c++) {
        if (c * 64 < a.R) {
          const int i = c * 64 + lane;
          const bool f = i < a.R && in_part(qs[c]);
          if (pp == 0 && i < a.R && (uint32_t)qs[c] >= nlim) a.drwt[trow * a.R + i] = 0.f;
          const uint64_t bal = __ballot(f);
          if (f) {
            const int pos = nr + __popcll(bal & below);
            sl[pos] = qs[c];
            wl[pos] = qw[c];
            ml[pos] = i << 8;
          }
          nr += __popcll(bal);
        }
      }
#pragma unroll
      for (int c = 0; c < MC; c++) {
        if (c * 64 < a.W) {
          const int i = c * 64 + lane;
          const bool f = i < a.W && in_part(ps[c]);
          if (pp == 0 && i < a.W && (uint32_t)ps[c] >= nlim) a.dwwt[trow * a.W + i] = 0.f;
          const uint64_t bal = __ballot(f);
          if (f) {
            const int pos = nr + nwr + __popcll(bal & below);
            sl[pos] = ps[c];
            wl[pos] = pw[c];
            ml[pos] = (i << 8) | kWrite;
          }
          nwr += __popcll(bal);
        }
      }
    }
    const int nev = nr + nwr;
    wave_lds_sync();
    const float al = nal, be = nbe;
    const float4 vv = nv;
    const float4 dO = ndO;
    prefetch(b - 1);  // in flight while this block is processed

    // ---- 2. hash: slot -> events of the block (bit 2*wave + kind) ---------
    // (a read whose bit is already set is a second read of that slot by the
    // same token)
    bool dupl = false;
    for (int e = lane; e < nev; e += 64) {
      const int32_t s = sl[e];
      const uint32_t bit = 1u << (2 * wave + ((ml[e] & kWrite) ? 1 : 0));
      const uint64_t mine = (uint64_t)(uint32_t)s | ((uint64_t)bit << 32);
      int p = (int)(mix32((uint32_t)s) & (uint32_t)hmsk);
      while (true) {
        const uint64_t old = atomicCAS(reinterpret_cast<unsigned long long*>(&htab[p]),
                                       (unsigned long long)kEmpty, (unsigned long long)mine);
        if (old == kEmpty) break;
        if ((int32_t)(uint32_t)old == s) {
          const uint64_t prev = atomicOr(reinterpret_cast<unsigned long long*>(&htab[p]),
                                         (unsigned long long)((uint64_t)bit << 32));
          if ((prev >> 32) & bit) dupl = true;
          break;
        }
        p = (p + 1) & hmsk;
      }
    }
    __syncthreads();  // hash complete (and the flags reset)

    // ---- 3. levels: block events on the slot that come earlier ------------
    int mylvl = 0;
    for (int e = lane; e < nev; e += 64) {
      const uint32_t m = probe(htab, hmsk, sl[e]);
      const int kind = (ml[e] & kWrite) ? 1 : 0;
      const int lvl = __popc(m & ((1u << (2 * wave + kind)) - 1u));
      ml[e] = (ml[e] & ~kLvl) | lvl;
      mylvl = max(mylvl, lvl);
    }
    wave_lds_sync();
    for (int o = 32; o > 0; o >>= 1) mylvl = max(mylvl, __shfl_xor(mylvl, o));
    const bool wdup = __ballot(dupl) != 0ull;
    if (lane == 0) {
      if (mylvl > 0) atomicMax(&s_maxl, mylvl);
      if (nev > CAPW) atomicOr(&s_ovf, 1);
      if (wdup) atomicOr(&s_ovf, 2);
    }
    __syncthreads();  // levels complete
    const int maxL = s_maxl;
    const bool ovf = s_ovf != 0;
    const bool dup = (s_ovf & 2) != 0;
    for (int i = tid; i < a.hsize; i += NT) htab[i] = kEmpty;  // lookups are done

    float4 dvacc = make_float4(0.f, 0.f, 0.f, 0.f);
    float accA = 0.f, accB = 0.f;

    // one event's adjoint from its rows: X = M_t row (read) or pre-write row
    // (write), D = dM row.  Dot products are reduced across the lane group by
    // every lane of the wave; `on` selects the lanes whose event it is.
    auto apply = [&](int e, bool on, float4 X, float4 D) {
      const int meta = on ? ml[e] : 0;
      const bool isw = (meta & kWrite) != 0;
      const float w = on ? wl[e] : 0.f;
      const float c = be * w;
      const float4 t1 = make_float4(vv.x - al * X.x, vv.y - al * X.y, vv.z - al * X.z,
                                    vv.w - al * X.w);
      // read: <dO, X>;  write: <G, v - alpha*old> and <G, old>
      const float d1 = group_sum<LPR>(on ? (isw ? dot4(D, t1) : dot4(dO, X)) : 0.f);
      const float d2 = group_sum<LPR>(on && isw ? dot4(D, X) : 0.f);
      if (!on) return;
      const int32_t s = sl[e];
      const int rank = meta >> 8;
      if (isw) {
        if (l == 0) a.dwwt[trow * a.W + rank] = be * d1;
        accB += w * d1;
        accA += (1.0f - c) * d2;
        dvacc = fma4(c, D, dvacc);
        const float k = (1.0f - c) * al;
        *reinterpret_cast<float4*>(dMst + (int64_t)s * a.d_v) = scale4(k, D);
        *reinterpret_cast<float4*>(Mst + (int64_t)s * a.d_v) = X;
      } else {
        if (l == 0) a.drwt[trow * a.R + rank] = d1;
        *reinterpret_cast<float4*>(dMst + (int64_t)s * a.d_v) = fma4(w, dO, D);
      }
    };
    // the rows event e needs (clamped to row 0 of the stream past the list)
    auto load_x = [&](int e, bool has) -> float4 {
      const int meta = has ? ml[e] : 0;
      const int32_t s = has ? sl[e] : 0;
      const float* p = (meta & kWrite)
                           ? a.tape + (trow * a.W + (meta >> 8)) * a.d_v + c0
                           : Mst + (int64_t)s * a.d_v;
      return *reinterpret_cast<const float4*>(p);
    };
    auto load_d = [&](int e, bool has) -> float4 {
      const int32_t s = has ? sl[e] : 0;
      return *reinterpret_cast<const float4*>(dMst + (int64_t)s * a.d_v);
    };

    if (!ovf) {
      // ---- 4. all events' rows, then level by level ------------------------
      float4 X[EPL], D[EPL];
#pragma unroll
      for (int i = 0; i < EPL; i++) {
        const int e = i * GPW + g;
        X[i] = load_x(e, e < nev);
        D[i] = load_d(e, e < nev);
      }
      for (int L = 0; L <= maxL; L++) {
        if (L > 0) {
#pragma unroll
          for (int i = 0; i < EPL; i++) {
            const int e = i * GPW + g;
            if (e < nev && (ml[e] & kLvl) == L) {
              X[i] = load_x(e, true);
              D[i] = load_d(e, true);
            }
          }
        }
#pragma unroll
        for (int i = 0; i < EPL; i++) {
          const int e = i * GPW + g;
          apply(e, e < nev && (ml[e] & kLvl) == L, X[i], D[i]);
        }
        if (L < maxL) __syncthreads();  // level-L stores before level-(L+1) loads
      }
    } else {
      // ---- 4'. serial: one wave at a time in processing order; a wave's
      // reads, then its writes (distinct slots).  Reads go in register-sized
      // chunks, or one at a time when a token of the block repeats a read
      // slot (lane group 0 takes each; a read's stores reach the row before
      // the next read's load) ----------------------------------------------
      for (int w = 0; w < kNW; w++) {
        if (wave == w) {
          if (dup) {
            for (int e = 0; e < nr; e++) {
              const bool mine = g == 0;
              const float4 X = load_x(e, mine);
              const float4 D = load_d(e, mine);
              apply(e, mine, X, D);
              __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
            }
          }
          for (int part = dup ? 1 : 0; part < 2; part++) {
            const int lo = part ? nr : 0, hi = part ? nev : nr;
            for (int base = lo; base < hi; base += CAPW) {
              float4 X[EPL], D[EPL];
#pragma unroll
              for (int i = 0; i < EPL; i++) {
                const int e = base + i * GPW + g;
                X[i] = load_x(e, e < hi);
                D[i] = load_d(e, e < hi);
              }
#pragma unroll
              for (int i = 0; i < EPL; i++) {
                const int e = base + i * GPW + g;
                apply(e, e < hi, X[i], D[i]);
              }
            }
            // the reads' stores before the writes' loads of the same slots
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
          }
        }
        __syncthreads();  // this wave's stores before the next wave's loads
      }
    }

    // ---- 5. per-token sums of the partition ---------------------------------
#pragma unroll
    for (int o = LPR; o < 64; o <<= 1) {
      dvacc = add4(dvacc, shfl_xor4(dvacc, o));
      accA += __shfl_xor(accA, o);
      accB += __shfl_xor(accB, o);
    }
    if (valid && g == 0) {
      if (a.P == 1) {
        *reinterpret_cast<float4*>(a.dv + trow * a.d_v + c0) = dvacc;
        if (l == 0) {
          a.dalpha[trow] = accA;
          a.dbeta[trow] = accB;
        }
      } else {
        const int64_t ST = (int64_t)a.S * a.T;
        *reinterpret_cast<float4*>(a.work + ((int64_t)pp * ST + trow) * a.d_v + c0) = dvacc;
        if (l == 0) {
          float* ab = a.work + (int64_t)a.P * ST * a.d_v;
          ab[((int64_t)pp * ST + trow) * 2] = accA;
          ab[((int64_t)pp * ST + trow) * 2 + 1] = accB;
        }
      }
    }
    __syncthreads();  // this block's stores before the next block's loads
  }
}

// dv = sum_p work_dv[p], (dalpha, dbeta) = sum_p work_ab[p], p ascending.
__global__ void __launch_bounds__(256) sdm_bwd_sum_kernel(const float* __restrict__ work,
                                                          float* __restrict__ dv,
                                                          float* __restrict__ dalpha,
                                                          float* __restrict__ dbeta,
                                                          int64_t ST, int d_v, int P) {
  const int64_t n4 = ST * d_v / 4;
  const float* ab = work + (int64_t)P * ST * d_v;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4 + ST; i += stride) {
    if (i < n4) {
      float4 s = reinterpret_cast<const float4*>(work)[i];
      for (int p = 1; p < P; p++) s = add4(s, reinterpret_cast<const float4*>(work)[p * n4 + i]);
      reinterpret_cast<float4*>(dv)[i] = s;
    } else {
      const int64_t t = i - n4;
      float x = ab[t * 2], y = ab[t * 2 + 1];
      for (int p = 1; p < P; p++) {
        x += ab[(p * ST + t) * 2];
        y += ab[(p * ST + t) * 2 + 1];
      }
      dalpha[t] = x;
      dbeta[t] = y;
    }
  }
}

template <int LPR, bool VBF16, int EPL, int MC>
hipError_t launch_bwd_t(const ScanBwdArgs& a, size_t lds, hipStream_t stream) {
  auto k = sdm_scan_bwd_kernel<LPR, VBF16, EPL, MC>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k, dim3(a.S * a.P), dim3(kNW * 64), lds, stream, a);
  return hipGetLastError();
}

}  // namespace

ScanBwdPlan plan_scan_bwd(int S, int T, int64_t N, int d_v, int W, int R) {
  ScanBwdPlan p{};
  p.lpr = d_v / 4;
  // partitions: one workgroup per CU (a workgroup holds 8 waves of up to 225
  // VGPRs, so a second one would not fit and would wait for a whole
  // sequence), while a token keeps >= 8 events in each partition
  int P = 1;
  while (P < 64 && (int64_t)S * (P * 2) <= kTargetWorkgroups && (W + R) / (P * 2) >= 8 &&
         P * 2 <= N)
    P *= 2;
  p.P = P;
  // registers: mean events of a token in one partition plus three standard
  // deviations; rarer tokens take the serial path, while every register slot
  // past a token's events is a padding load
  const double mean = (double)(W + R) / P;
  const double need = mean + 3.0 * sqrt(mean * (1.0 - 1.0 / P));
  const int gpw = 64 / p.lpr;
  p.epl = need <= 4 * gpw ? 4 : need <= 8 * gpw ? 8 : need <= 12 * gpw ? 12 : 16;
  int64_t hs = 1;
  while (hs < 2LL * kNW * (W + R)) hs *= 2;
  p.hsize = (int)hs;
  p.lcap = W + R;
  p.lds = (size_t)p.hsize * 8 + (size_t)kNW * p.lcap * 12;
  p.work_bytes = P > 1 ? (size_t)P * S * T * (d_v + 2) * sizeof(float) : 0;
  return p;
}

hipError_t launch_scan_bwd(const ScanBwdArgs& a0, const ScanBwdPlan& p, bool vbf16,
                           hipStream_t stream) {
  ScanBwdArgs a = a0;
  a.P = p.P;
  a.hsize = p.hsize;
  a.lcap = p.lcap;
  a.xcd_map = ((int64_t)a.S * a.P) % 8 == 0 ? 1 : 0;
  if (a.T == 0) return hipSuccess;
  hipError_t e;
  const int kmax = a.W > a.R ? a.W : a.R;
  const int mc = kmax <= 64 ? 1 : kmax <= 128 ? 2 : 4;
#define SDM_BWD_CASE(LPR_, EPL_, MC_)                                     \
  if (p.lpr == LPR_ && p.epl == EPL_ && mc == MC_) {                      \
    e = vbf16 ? launch_bwd_t<LPR_, true, EPL_, MC_>(a, p.lds, stream)     \
              : launch_bwd_t<LPR_, false, EPL_, MC_>(a, p.lds, stream);   \
  } else
#define SDM_BWD_MC(LPR_, EPL_) \
  SDM_BWD_CASE(LPR_, EPL_, 1) SDM_BWD_CASE(LPR_, EPL_, 2) SDM_BWD_CASE(LPR_, EPL_, 4)
#define SDM_BWD_EPL(LPR_) \
  SDM_BWD_MC(LPR_, 4) SDM_BWD_MC(LPR_, 8) SDM_BWD_MC(LPR_, 12) SDM_BWD_MC(LPR_, 16)
  SDM_BWD_EPL(4)
  SDM_BWD_EPL(8)
  SDM_BWD_EPL(16)
  SDM_BWD_EPL(32)
  SDM_BWD_EPL(64) { return hipErrorInvalidValue; }
#undef SDM_BWD_EPL
#undef SDM_BWD_MC
#undef SDM_BWD_CASE
  if (e != hipSuccess) return e;
  if (p.P > 1) {
    const int64_t ST = (int64_t)a.S * a.T;
    const int64_t n = ST * a.d_v / 4 + ST;
    int grid = (int)((n + 255) / 256);
    if (grid > 4096) grid = 4096;
    hipLaunchKernelGGL(sdm_bwd_sum_kernel, dim3(grid), dim3(256), 0, stream, a.work, a.dv,
                       a.dalpha, a.dbeta, ST, a.d_v, p.P);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace sdm
