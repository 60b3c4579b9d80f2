// The sequential sparse gated-delta scan kernel for gfx950, shared by its two
// builds: scan.hip (plain row loads, planner and launch) and scan_buf.hip
// (buffer-form row loads).
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
//   - slot partition  : rows whose slot hash falls in partition p (a hash, not
//                       slot bits: product-key slots of one token share
//                       sub-key indices, so their low bits are far from
//                       uniform).  A token's events are split across the P
//                       partitions; each partition workgroup
//                       produces a partial read sum, added in partition order
//                       by sdm_partial_sum_kernel.
// One workgroup owns one (stream, slice, partition) and walks all tokens.
//
// Inside a workgroup, tokens go in blocks of NW tokens, one wave per token.
// Block b's rows are loaded during block b-1, right after block b-1's last
// stores (a barrier orders them), so every load sees the state before block
// b; their latency overlaps block b's own set-up (hash build, dependence
// levels, two barriers), which issues no memory operation.  The indices of
// block b+1 are prefetched one block earlier still.  In-block dependences
// come from an LDS hash of the block's write slots (slot -> bitmask of
// writing tokens):
//   write at token u of slot s : level = #{block writers of s before u}
//   read  at token u of slot s : level = #{block writers of s at or before u}
// Level-0 events use the loaded rows; level-L events (L >= 1) reload after
// the level-(L-1) stores (barrier), and all loads of a level come before its
// stores (a level-L read of s must not see the level-L write of s by a later
// token).  Writes of one slot get distinct levels, so a level never races
// with itself.  Reads are summed after all levels in fixed event order, so
// the output does not depend on where blocks start.
//
// Memory operations on the common path are unconditional (clamped or dummy
// addresses) and issued oldest-needed first, so the compiler's in-order wait
// counts are exact and never drain loads that are still meant to be in
// flight.
//
// gfx950 workgroup memory ordering: all waves of a workgroup share the CU's
// in-order vector L1, and __syncthreads() (workgroup-scope release/acquire)
// orders a wave's earlier global stores before another wave's later global
// loads, without draining the stores.  A load issued before a barrier cannot
// see a store issued after it.
#pragma once
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <algorithm>

#include "sdm_internal.h"
#include "scan_common.h"

namespace sdm {

using namespace scanc;

namespace {

constexpr int kLevel = 0x7f;

// Buffer resource of a stream's table: byte offsets are 32-bit, so the
// buffer form is used only when the table spans at most kBufMaxBytes, and an
// offset of kBufPastEnd is then always out of range.  Word 3 is the gfx9
// family's raw-buffer format (32-bit data, no swizzle).
constexpr int64_t kBufMaxBytes = int64_t{1} << 31;
constexpr uint32_t kBufPastEnd = 0x80000000u;
constexpr int kBufWord3 = 0x00020000;

__device__ __forceinline__ float4 buffer_load4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  typedef unsigned int u4 __attribute__((ext_vector_type(4)));
  const u4 x = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
  return make_float4(__uint_as_float(x.x), __uint_as_float(x.y), __uint_as_float(x.z),
                     __uint_as_float(x.w));
}

// write strength c = beta*w and 1 - c, each rounded separately
__device__ __forceinline__ void gate(float beta, float w, float& c, float& omc) {
#pragma clang fp contract(off)
  c = beta * w;
  omc = 1.0f - c;
}

// Gated delta update of one element: (1-c)*(a*m) + c*v, each product and the
// sum rounded separately (no contraction), so c == 1 gives v, c == 0 gives a*m.
__device__ __forceinline__ float upd(float m, float a, float omc, float c, float v) {
#pragma clang fp contract(off)
  const float mt = a * m;
  const float keep = omc * mt;
  const float put = c * v;
  return keep + put;
}

__device__ __forceinline__ float4 upd4(float4 m, float a, float omc, float c, float4 v) {
  return make_float4(upd(m.x, a, omc, c, v.x), upd(m.y, a, omc, c, v.y),
                     upd(m.z, a, omc, c, v.z), upd(m.w, a, omc, c, v.w));
}

}  // namespace

// LPR: lanes per row slice (CW = 4*LPR columns).  NW: waves = tokens per block.
// MC: 64-wide chunks of a token's index list (W, R <= 64*MC).  EPL: events per
// lane group held in registers (a wave holds EPL*64/LPR events).  TAPE: also
// store every write event's row as it was before the write (the values the
// reverse sweep of the gradient needs) at tape[stream][t][rank].  BUF: the
// speculative row loads are buffer loads relative to the stream's table
// (which then spans at most 2^31 bytes), so that a load past an event list
// takes an offset beyond the table's end: the hardware answers it with zeros
// and sends no request to memory.
template <int LPR, bool VBF16, int NW, int MC, int EPL, bool TAPE, bool BUF>
__global__ void __launch_bounds__(NW * 64, 1) sdm_scan_kernel(ScanArgs a) {
  constexpr int GPW = 64 / LPR;    // lane groups per wave
  constexpr int CAPW = GPW * EPL;  // events per wave held in registers
  constexpr int CW = 4 * LPR;
  constexpr int NT = NW * 64;

  extern __shared__ __align__(16) unsigned char smem[];
  uint64_t* htab = reinterpret_cast<uint64_t*>(smem);              // [hsize]
  int32_t* lslot = reinterpret_cast<int32_t*>(htab + a.hsize);     // [NW][lcap]
  float* lwt = reinterpret_cast<float*>(lslot + NW * a.lcap);      // [NW][lcap]
  int32_t* lmeta = reinterpret_cast<int32_t*>(lwt + NW * a.lcap);  // [NW][lcap]
  __shared__ int s_flag[3][2];  // per block (index mod 3): max level, overflow

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
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
  const int nblk = (a.T + NW - 1) / NW;
  const int hmsk = a.hsize - 1;
  float* Mst = a.M + (int64_t)st * a.N * a.d_v + c0;
  int32_t* sl = lslot + wave * a.lcap;  // this wave's event list
  float* wl = lwt + wave * a.lcap;
  int32_t* ml = lmeta + wave * a.lcap;

  auto row = [&](int32_t s) -> float* { return Mst + (int64_t)s * a.d_v; };
  // pre-write row of write event e of this wave's token (row `trow` of [S*T])
  auto record = [&](int64_t trow, int e, const float4& x) {
    if constexpr (TAPE)
      *reinterpret_cast<float4*>(a.tape + (trow * a.W + (ml[e] >> 8)) * a.d_v + c0) = x;
  };
  // an event whose slot lies outside [0, N) belongs to no partition: it is
  // neither read nor written
  const uint32_t nlim = (uint32_t)a.N;
  auto in_part = [&](int32_t s) {
    return (uint32_t)s < nlim && ((mix32((uint32_t)s) >> 16) & pmask) == (uint32_t)pp;
  };

  // ---- index prefetch for one token (registers; unconditional loads) -----
  int32_t ps[MC], qs[MC];
  float pw[MC], qw[MC];
  bool pok = false;  // the prefetched token exists
  auto prefetch = [&](int blk) {
    const int tok = blk * NW + wave;
    pok = blk < nblk && tok < a.T;
    const int64_t trow = (int64_t)st * a.T + (pok ? tok : 0);
#pragma unroll
    for (int c = 0; c < MC; c++) {
      const int i = c * 64 + lane;
      const int iw = i < a.W ? i : a.W - 1, ir = i < a.R ? i : a.R - 1;
      ps[c] = a.widx[trow * a.W + iw];
      pw[c] = a.wwt[trow * a.W + iw];
      qs[c] = a.ridx[trow * a.R + ir];
      qw[c] = a.rwt[trow * a.R + ir];
    }
  };
  // the prefetched token's events of this partition into the wave's list:
  // writes first, then reads, each in rank order
  auto compact = [&](int& nw, int& nr) {
    const uint64_t below = (1ull << lane) - 1ull;
    nw = 0;
#pragma unroll
    for (int c = 0; c < MC; c++) {
      if (c * 64 < a.W) {
        const bool f = pok && c * 64 + lane < a.W && in_part(ps[c]);
        const uint64_t bal = __ballot(f);
        if (f) {
          const int pos = nw + __popcll(bal & below);
          sl[pos] = ps[c];
          wl[pos] = pw[c];
          if constexpr (TAPE) ml[pos] = (c * 64 + lane) << 8;  // rank in the token's list
        }
        nw += __popcll(bal);
      }
    }
    nr = 0;
#pragma unroll
    for (int c = 0; c < MC; c++) {
      if (c * 64 < a.R) {
        const bool f = pok && c * 64 + lane < a.R && in_part(qs[c]);
        const uint64_t bal = __ballot(f);
        if (f) {
          const int pos = nw + nr + __popcll(bal & below);
          sl[pos] = qs[c];
          wl[pos] = qw[c];
        }
        nr += __popcll(bal);
      }
    }
  };
  // gates and this lane's slice of v for the wave's token of block blk
  // (clamped, always loaded)
  auto gates = [&](int blk, float& al, float& be, float4& vv) {
    const int tok = blk * NW + wave;
    const int64_t tr = (int64_t)st * a.T + (tok < a.T ? tok : 0);
    al = a.alpha[tr];
    be = a.beta[tr];
    vv = load_v4(a.v, VBF16, tr * a.d_v + c0);
  };
  // every lane always issues EPL row loads; positions past the list read
  // nothing (BUF: an offset past the table) or row 0 of the stream (one cache
  // line per instruction, never used)
  const __amdgpu_buffer_rsrc_t mrs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.M + (int64_t)st * a.N * a.d_v), (short)0,
      (int)(uint32_t)std::min<int64_t>(a.N * a.d_v * 4, kBufMaxBytes), kBufWord3);
  auto issue = [&](int ne, float4(&x)[EPL]) {
#pragma unroll
    for (int i = 0; i < EPL; i++) {
      const int e = i * GPW + g;
      if constexpr (BUF) {
        const uint32_t off =
            e < ne ? ((uint32_t)sl[e] * (uint32_t)a.d_v + (uint32_t)c0) * 4u : kBufPastEnd;
        x[i] = buffer_load4(mrs, off);
      } else {
        x[i] = *reinterpret_cast<const float4*>(row(e < ne ? sl[e] : 0));
      }
    }
  };

  // ---- set-up: empty hash, clear flags, block 0 in flight ----------------
  for (int i = tid; i < a.hsize; i += NT) htab[i] = kEmpty;
  if (tid < 6) s_flag[tid / 2][tid % 2] = 0;
  __syncthreads();
  float4 X[EPL];
  int nwc = 0, nrc = 0;
  float gA, gB;
  float4 gV;
  prefetch(0);
  compact(nwc, nrc);
  wave_lds_sync();
  gates(0, gA, gB, gV);
  prefetch(1);
  {
    const bool fit = nwc + nrc <= CAPW;
    issue(fit ? nwc + nrc : 0, X);
    if (!fit && lane == 0) atomicOr(&s_flag[0][1], 1);
  }

  for (int b = 0; b < nblk; b++) {
    const int fcur = b % 3, fnext = (b + 1) % 3, fprev = (b + 2) % 3;
    const int tok = b * NW + wave;
    const bool valid = tok < a.T;
    const int64_t trow = (int64_t)st * a.T + tok;
    const int nec = nwc + nrc;
    const float alpha = gA, beta = gB;
    const float4 vv = gV;

    // ---- 1. block b's writers into the hash ------------------------------
    for (int e = lane; e < nwc; e += 64) {
      const int32_t s = sl[e];
      const uint64_t mine = (uint64_t)(uint32_t)s | ((uint64_t)(1u << wave) << 32);
      int p = (int)(mix32((uint32_t)s) & (uint32_t)hmsk);
      while (true) {
        const uint64_t old = atomicCAS(reinterpret_cast<unsigned long long*>(&htab[p]),
                                       (unsigned long long)kEmpty, (unsigned long long)mine);
        if (old == kEmpty) break;
        if ((int32_t)(uint32_t)old == s) {
          atomicOr(reinterpret_cast<unsigned long long*>(&htab[p]),
                   (unsigned long long)((uint64_t)(1u << wave) << 32));
          break;
        }
        p = (p + 1) & hmsk;
      }
    }
    __syncthreads();  // BAR1: block b's hash complete
    if (tid == 0) s_flag[fprev][0] = 0, s_flag[fprev][1] = 0;  // block b-1's flags

    // ---- 2. dependence levels --------------------------------------------
    int mylvl = 0;
    const uint32_t wbefore = (1u << wave) - 1u;  // writers strictly before
    const uint32_t rbefore = (2u << wave) - 1u;  // writers at or before
    for (int e = lane; e < nec; e += 64) {
      const uint32_t m = probe(htab, hmsk, sl[e]);
      const int lvl = __popc(m & (e < nwc ? wbefore : rbefore));
      if constexpr (TAPE)
        ml[e] = e < nwc ? ((ml[e] & ~kLevel) | lvl) : lvl;
      else
        ml[e] = lvl;
      mylvl = max(mylvl, lvl);
    }
    wave_lds_sync();  // levels written by other lanes are read below
    for (int o = 32; o > 0; o >>= 1) mylvl = max(mylvl, __shfl_xor(mylvl, o));
    if (lane == 0 && mylvl > 0) atomicMax(&s_flag[fcur][0], mylvl);
    __syncthreads();  // BAR2: levels of block b complete
    const int maxL = s_flag[fcur][0];
    const bool ovf = s_flag[fcur][1] != 0;

    // ---- 3. level 0 (and, without dependences, the reads) -----------------
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    if (!ovf) {
#pragma unroll
      for (int i = 0; i < EPL; i++) {
        const int e = i * GPW + g;
        if (e < nwc && (ml[e] & kLevel) == 0) {
          float c, omc;
          gate(beta, wl[e], c, omc);
          *reinterpret_cast<float4*>(row(sl[e])) = upd4(X[i], alpha, omc, c, vv);
          record(trow, e, X[i]);
        }
      }
      if (maxL == 0) {
#pragma unroll
        for (int i = 0; i < EPL; i++) {
          const int e = i * GPW + g;
          if (e >= nwc && e < nec) acc = fma4(wl[e], X[i], acc);
        }
      }
    }
    for (int i = tid; i < a.hsize; i += NT) htab[i] = kEmpty;  // lookups are done
    __syncthreads();  // BAR_A: level-0 stores before any later load

    // ---- 4. dependent levels ---------------------------------------------
    if (!ovf && maxL > 0) {
      for (int L = 1; L <= maxL; L++) {
#pragma unroll
        for (int i = 0; i < EPL; i++) {
          const int e = i * GPW + g;
          if (e < nec && (ml[e] & kLevel) == L) X[i] = *reinterpret_cast<const float4*>(row(sl[e]));
        }
        __syncthreads();  // every level-L load issued before any level-L store
#pragma unroll
        for (int i = 0; i < EPL; i++) {
          const int e = i * GPW + g;
          if (e < nwc && (ml[e] & kLevel) == L) {
            float c, omc;
            gate(beta, wl[e], c, omc);
            *reinterpret_cast<float4*>(row(sl[e])) = upd4(X[i], alpha, omc, c, vv);
            record(trow, e, X[i]);
          }
        }
        __syncthreads();  // level-L stores before level-(L+1) loads
      }
      // every read row now holds the value its token must see: sum them in
      // event order, so the result does not depend on where blocks start
#pragma unroll
      for (int i = 0; i < EPL; i++) {
        const int e = i * GPW + g;
        if (e >= nwc && e < nec) acc = fma4(wl[e], X[i], acc);
      }
    } else if (ovf) {
      // overflow path: some token has more events than fit in registers.  Per
      // level: all reads (chunked, no stores), barrier, all writes (chunked;
      // writes of one level never share a slot), barrier.
      for (int L = 0; L <= maxL; L++) {
        for (int base = nwc; base < nec; base += CAPW) {
#pragma unroll
          for (int i = 0; i < EPL; i++) {
            const int e = base + i * GPW + g;
            if (e < nec && (ml[e] & kLevel) == L) X[i] = *reinterpret_cast<const float4*>(row(sl[e]));
          }
#pragma unroll
          for (int i = 0; i < EPL; i++) {
            const int e = base + i * GPW + g;
            if (e < nec && (ml[e] & kLevel) == L) acc = fma4(wl[e], X[i], acc);
          }
        }
        __syncthreads();  // level-L reads done before level-L writes store
        for (int base = 0; base < nwc; base += CAPW) {
#pragma unroll
          for (int i = 0; i < EPL; i++) {
            const int e = base + i * GPW + g;
            if (e < nwc && (ml[e] & kLevel) == L) X[i] = *reinterpret_cast<const float4*>(row(sl[e]));
          }
#pragma unroll
          for (int i = 0; i < EPL; i++) {
            const int e = base + i * GPW + g;
            if (e < nwc && (ml[e] & kLevel) == L) {
              float c, omc;
              gate(beta, wl[e], c, omc);
              *reinterpret_cast<float4*>(row(sl[e])) = upd4(X[i], alpha, omc, c, vv);
              record(trow, e, X[i]);
            }
          }
        }
        __syncthreads();  // level-L stores before level-(L+1) loads
      }
    }

    // ---- 5. read sum across the wave's lane groups (fixed order) ----------
#pragma unroll
    for (int o = LPR; o < 64; o <<= 1) acc = add4(acc, shfl_xor4(acc, o));
    if (valid && g == 0) {
      float* dst = a.P == 1 ? a.out + trow * a.d_v + c0
                            : a.work + ((int64_t)pp * a.S * a.T + trow) * a.d_v + c0;
      // streamed past the caches (read once, by the partial sum) so that they
      // do not displace table rows
      __builtin_nontemporal_store(acc.x, dst + 0);
      __builtin_nontemporal_store(acc.y, dst + 1);
      __builtin_nontemporal_store(acc.z, dst + 2);
      __builtin_nontemporal_store(acc.w, dst + 3);
    }

    // ---- 6. next block: compact, gates, indices after it, then its rows ---
    // (every store of block b precedes these loads: the last barrier above
    // follows the last store)
    int nwn = 0, nrn = 0;
    if (b + 1 < nblk) compact(nwn, nrn);
    wave_lds_sync();
    gates(b + 1, gA, gB, gV);
    prefetch(b + 2);
    const bool fit = nwn + nrn <= CAPW;
    issue(fit ? nwn + nrn : 0, X);
    if (b + 1 < nblk && !fit && lane == 0) atomicOr(&s_flag[fnext][1], 1);
    nwc = nwn;
    nrc = nrn;
  }
}

// ----------------------------------------------------------------- launch --

template <int LPR, bool VBF16, int NW, int MC, int EPL, bool BUF>
hipError_t launch_scan_t(const ScanArgs& a, size_t lds, hipStream_t stream) {
  auto k = sdm_scan_kernel<LPR, VBF16, NW, MC, EPL, false, BUF>;
  if constexpr (NW > 1) {  // one-wave blocks are planned only without a tape
    if (a.tape) k = sdm_scan_kernel<LPR, VBF16, NW, MC, EPL, true, BUF>;
  }
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k, dim3(a.S * a.CS * a.P), dim3(NW * 64), lds, stream, a);
  return hipGetLastError();
}

// the scan kernel for this plan (buffer-form row loads or plain ones)
template <bool BUF>
hipError_t launch_scan_kernel(const ScanArgs& a, const ScanPlan& p, bool vbf16,
                              hipStream_t stream) {
  hipError_t e;
  const int mc = (a.W > a.R ? a.W : a.R) <= 64 ? 1 : ((a.W > a.R ? a.W : a.R) <= 128 ? 2 : 4);
#define SDM_SCAN_CASE(LPR_, MC_, EPL_)                                                \
  if (p.lpr == LPR_ && mc == MC_ && p.epl == EPL_) {                                  \
    if (p.nw == 1)                                                                    \
      e = vbf16 ? launch_scan_t<LPR_, true, 1, MC_, EPL_, BUF>(a, p.lds, stream)      \
                : launch_scan_t<LPR_, false, 1, MC_, EPL_, BUF>(a, p.lds, stream);    \
    else                                                                              \
      e = vbf16 ? launch_scan_t<LPR_, true, 8, MC_, EPL_, BUF>(a, p.lds, stream)      \
                : launch_scan_t<LPR_, false, 8, MC_, EPL_, BUF>(a, p.lds, stream);    \
  } else
#define SDM_SCAN_EPL(LPR_, MC_) \
  SDM_SCAN_CASE(LPR_, MC_, 8) SDM_SCAN_CASE(LPR_, MC_, 12) SDM_SCAN_CASE(LPR_, MC_, 16)
  SDM_SCAN_EPL(16, 1)
  SDM_SCAN_EPL(16, 2)
  SDM_SCAN_EPL(16, 4)
  SDM_SCAN_EPL(8, 1)
  SDM_SCAN_EPL(8, 2)
  SDM_SCAN_EPL(8, 4)
  SDM_SCAN_EPL(4, 1)
  SDM_SCAN_EPL(4, 2)
  SDM_SCAN_EPL(4, 4) { return hipErrorInvalidValue; }
#undef SDM_SCAN_EPL
#undef SDM_SCAN_CASE
  return e;
}

// defined in scan_buf.hip (the buffer-form kernels, compiled on their own)
hipError_t launch_scan_kernel_buf(const ScanArgs& a, const ScanPlan& p, bool vbf16,
                                  hipStream_t stream);

}  // namespace sdm
