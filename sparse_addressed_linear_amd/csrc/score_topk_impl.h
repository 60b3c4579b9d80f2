// Kernel templates of the product-key addressing (included by the score_topk*.hip units).
#pragma once
// Product-key addressing for Sparse Delta Memory, for gfx950.
//
// Method ("Sparse Delta Memory", gist.science summaries of paper 2607.07386;
// Spanish page "Mecanismo Central" item 2, French page "Mecanisme Central"):
// the projected key (query) is cut into two halves; each half is scored
// against its own table of n_sub sub-keys (product-key memory); slot
// s = i*n_sub + j scores s1[i] + s2[j]; the top-W (top-R) slots are found
// through topk(s1 (+) s2) = topk(topk(s1) (+) topk(s2)) without forming the
// N = n_sub^2 scores.  Weights: softmax over the selected sums.  Order: score
// descending, ties to the lower index (sub-key index in stage 1, slot in
// stage 2).
//
// One workgroup handles kTT tokens of one (b,h) stream:
//   1. half scores for the tile: bf16 -> MFMA v_mfma_f32_16x16x32_bf16
//      (sub-keys x tokens, fp32 accumulate), fp32 -> plain VALU dot products
//      in the same sequential order as a scalar loop; results to LDS.
//   2. stage 1, one wave per (token, half): exact top-m selection.
//   3. stage 2, one wave per token: top-k of the outer sums over the pruned
//      rank grid {(a,b): (a+1)(b+1) <= k} -- a pair outside it is beaten by at
//      least k pairs of its dominating rectangle.  With ties in the fp32 sums
//      that argument can fail, so the best pair just outside the grid is
//      checked and, if it could compete, the full m x m grid is ranked.
// Exact selection of the k best of n values held by one wave: every value
// becomes a unique 64-bit key (order-preserving score bits, then the
// complemented index), a threshold t with k <= #{key >= t} <= cap is found by
// counting with ballots (first guess from the score distribution, then integer
// bisection on keys, which always terminates because keys are unique), the
// keys >= t are compacted to LDS and sorted by a register bitonic network.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "sdm_internal.h"

namespace sdm {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kTT = 8;       // tokens per workgroup (MFMA tiles carry 16 columns)
constexpr int kWaves = 8;    // waves per workgroup
constexpr int kThreads = kWaves * 64;
constexpr int kCapMax = 256; // largest candidate set sorted at once
constexpr int kGridMax = 1024;  // largest pruned grid held in registers

__device__ __forceinline__ uint32_t ord32(float s) {
  uint32_t u = __float_as_uint(s);
  if ((u << 1) == 0u) u = 0u;  // -0 ranks equal to +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float unord32(uint32_t o) {
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}

// larger key = ranks ahead: higher score, then lower index
__device__ __forceinline__ uint64_t make_key(float s, uint32_t id) {
  return ((uint64_t)ord32(s) << 32) | (uint64_t)(0xffffffffu - id);
}
__device__ __forceinline__ float key_score(uint64_t k) { return unord32((uint32_t)(k >> 32)); }
__device__ __forceinline__ uint32_t key_id(uint64_t k) { return 0xffffffffu - (uint32_t)k; }

// sum over e ascending of x[e]*c[e], each product and sum rounded in fp32
__device__ __forceinline__ float dot_seq(const float* x, const float* c, int n) {
#pragma clang fp contract(off)
  float acc = 0.f;
  for (int e = 0; e < n; e++) {
    const float p = x[e] * c[e];
    acc = acc + p;
  }
  return acc;
}

__device__ __forceinline__ float wave_sum(float x) {
  const int lane = __lane_id();
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += xor_shuffle(x, o, lane);
  return x;
}
__device__ __forceinline__ uint64_t wave_max64(uint64_t x) {
  const int lane = __lane_id();
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const uint64_t y = xor_shuffle(x, o, lane);
    x = y > x ? y : x;
  }
  return x;
}

template <int NPL>
__device__ __forceinline__ int count_ge(const uint64_t (&key)[NPL], uint64_t t) {
  int c = 0;
#pragma unroll
  for (int j = 0; j < NPL; j++) c += __popcll(__ballot(key[j] >= t));
  return c;
}

// Threshold t with k <= #{key >= t} <= cap.  Requires #{key >= lo} >= k and
// #{key >= hi} < k.  Keys are unique, so bisection ends with #{key >= t} == k
// at the latest.
template <int NPL>
__device__ uint64_t find_threshold(const uint64_t (&key)[NPL], int k, int cap, uint64_t guess,
                                   uint64_t lo, uint64_t hi) {
  uint64_t t = (guess > lo && guess < hi) ? guess : lo + (hi - lo) / 2;
  for (int it = 0; it < 96; it++) {
    const int c = count_ge(key, t);
    if (c >= k && c <= cap) return t;
    if (c < k) hi = t;
    else lo = t;
    if (hi - lo <= 1) return lo;
    t = lo + (hi - lo) / 2;
  }
  return lo;
}

// Ascending-index bitonic network over 64*E keys held E per lane (element
// i = lane*E + r), sorting into DESCENDING order.
template <int E>
__device__ __forceinline__ void bitonic_desc(uint64_t (&v)[E], int lane) {
#pragma unroll
  for (int s = 2; s <= 64 * E; s <<= 1) {
#pragma unroll
    for (int j = s >> 1; j > 0; j >>= 1) {
      if (j >= E) {
#pragma unroll
        for (int r = 0; r < E; r++) {
          const uint64_t o = xor_shuffle(v[r], j / E, lane);
          const int i = lane * E + r;
          const bool lower = (i & j) == 0;
          const bool desc = (i & s) == 0;
          const bool keep_max = lower == desc;
          v[r] = keep_max ? (o > v[r] ? o : v[r]) : (o < v[r] ? o : v[r]);
        }
      } else {
#pragma unroll
        for (int r = 0; r < E; r++) {
          if ((r & j) == 0) {
            const int i = lane * E + r;
            const bool desc = (i & s) == 0;
            const uint64_t p = v[r], q = v[r | j];
            const bool swap = desc ? (q > p) : (q < p);
            v[r] = swap ? q : p;
            v[r | j] = swap ? p : q;
          }
        }
      }
    }
  }
}

// Sort the c (<= kCapMax) keys in buf descending; lanes then write the first k
// through `emit(rank, key)`.
template <int E, typename Emit>
__device__ __forceinline__ void sort_emit_e(uint64_t* buf, int c, int k, int lane, Emit emit) {
  uint64_t v[E];
#pragma unroll
  for (int r = 0; r < E; r++) {
    const int i = lane * E + r;
    v[r] = i < c ? buf[i] : 0ull;
  }
  bitonic_desc<E>(v, lane);
#pragma unroll
  for (int r = 0; r < E; r++) {
    const int i = lane * E + r;
    if (i < k) emit(i, v[r]);
  }
}

template <typename Emit>
__device__ __forceinline__ void sort_emit(uint64_t* buf, int c, int k, int lane, Emit emit) {
  if (c <= 64) sort_emit_e<1>(buf, c, k, lane, emit);
  else if (c <= 128) sort_emit_e<2>(buf, c, k, lane, emit);
  else sort_emit_e<4>(buf, c, k, lane, emit);
}

// Compact keys >= t into buf (ballot order); returns the count.
template <int NPL>
__device__ __forceinline__ int compact_ge(const uint64_t (&key)[NPL], uint64_t t, uint64_t* buf,
                                          int lane) {
  int base = 0;
  const uint64_t below = (1ull << lane) - 1ull;
#pragma unroll
  for (int j = 0; j < NPL; j++) {
    const bool f = key[j] >= t;
    const uint64_t m = __ballot(f);
    if (f) buf[base + __popcll(m & below)] = key[j];
    base += __popcll(m);
  }
  return base;
}

// Exact top-k of the NPL*64 keys of one wave (unused entries hold key 0 and
// never outrank a real one), delivered in rank order through emit.
// `guess` is a first threshold estimate (0 = none).
template <int NPL, typename Emit>
__device__ void wave_topk(const uint64_t (&key)[NPL], int k, uint64_t guess, uint64_t* buf,
                          int lane, Emit emit) {
  uint64_t mx = 0;
#pragma unroll
  for (int j = 0; j < NPL; j++) mx = key[j] > mx ? key[j] : mx;
  mx = wave_max64(mx);
  const int cap = min(kCapMax, max(64, 2 * k));
  const uint64_t t = find_threshold(key, k, cap, guess, 0ull, mx + 1ull);
  const int c = compact_ge(key, t, buf, lane);
  wave_lds_sync();
  sort_emit(buf, c, k, lane, emit);
  wave_lds_sync();
}

}  // namespace

// Shared-memory layout (bytes), n_sub and m known at launch.
struct ScoreSmem {
  size_t sc, ls, li, cbuf, grid, rowoff, total;
};

__host__ __device__ inline ScoreSmem score_smem(int n_sub, int m) {
  ScoreSmem s;
  size_t o = 0;
  s.sc = o;     o += (size_t)kTT * (n_sub + 4) * 4;  // rows padded: fewer LDS bank conflicts
  s.ls = o;     o += (size_t)2 * kTT * m * 4;
  s.li = o;     o += (size_t)2 * kTT * m * 4;
  o = (o + 15) & ~(size_t)15;
  s.cbuf = o;   o += (size_t)kWaves * (m * 2 > 64 ? m * 2 : 64) * 8;  // 2k keys per wave
  s.grid = o;   o += (size_t)kGridMax * 4;
  s.rowoff = o; o += (size_t)(m + 1) * 4;
  s.total = o;
  return s;
}

// Half scores of kTT tokens against all n_sub sub-keys of one half, on MFMA:
// D[sub-key][token] = sum_k C[sub-key][k] * x[token][k], 16x16 tiles of
// v_mfma_f32_16x16x32_bf16.  A wave owns sub-key tiles i0 = 16*wave + 128*j;
// the sub-key fragments of TB tiles are loaded together, so one L2 round trip
// covers TB tiles.
template <int KS>
__device__ __forceinline__ void mfma_half_scores(const uint16_t* Xb, const uint16_t* Cb,
                                                 int n_sub, int dh, float* sc, int scs,
                                                 int wave, int lane, bool tok_ok) {
  constexpr int TB = 8 / KS;   // tiles per batch
  const int tl = lane & 15;    // token (B column) / sub-key (A row) in the tile
  const int kq = lane >> 4;    // which 8-wide K chunk of the 32
  bf16x8 bfrag[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ks++) {
    const int d0 = ks * 32 + kq * 8;
    bfrag[ks] = (tok_ok && d0 < dh) ? *reinterpret_cast<const bf16x8*>(Xb + d0) : bf16x8{};
  }
  for (int ib = wave * 16; ib < n_sub; ib += kWaves * 16 * TB) {
    bf16x8 af[TB][KS];
#pragma unroll
    for (int t = 0; t < TB; t++) {
      const int sk = ib + t * kWaves * 16 + tl;
#pragma unroll
      for (int ks = 0; ks < KS; ks++) {
        const int d0 = ks * 32 + kq * 8;
        af[t][ks] = (sk < n_sub && d0 < dh)
                        ? *reinterpret_cast<const bf16x8*>(Cb + (int64_t)sk * dh + d0)
                        : bf16x8{};
      }
    }
#pragma unroll
    for (int t = 0; t < TB; t++) {
      floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ks++)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[t][ks], bfrag[ks], acc, 0, 0, 0);
      // D[row = sub-key i0 + 4*kq + r][col = token tl]
      const int s0 = ib + t * kWaves * 16 + 4 * kq;
      if (tok_ok && s0 < n_sub) {
        if (s0 + 3 < n_sub) {
          *reinterpret_cast<float4*>(sc + tl * scs + s0) = make_float4(acc[0], acc[1], acc[2], acc[3]);
        } else {
          for (int r = 0; r < 4 && s0 + r < n_sub; r++) sc[tl * scs + s0 + r] = acc[r];
        }
      }
    }
  }
}

template <bool BF16, int NPL1, int NPL2>
__global__ void __launch_bounds__(kThreads, 4) sdm_score_topk_kernel(ScoreArgs a, float zW,
                                                                    float zR) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int n_sub = a.n_sub;
  const int mmax = max(a.W, a.R);
  const ScoreSmem L = score_smem(n_sub, mmax);
  float* sc = reinterpret_cast<float*>(smem + L.sc);       // [kTT][n_sub + 4]
  const int scs = n_sub + 4;
  float* ls = reinterpret_cast<float*>(smem + L.ls);       // [2][kTT][mmax]
  int32_t* li = reinterpret_cast<int32_t*>(smem + L.li);   // [2][kTT][mmax]
  uint64_t* cbufs = reinterpret_cast<uint64_t*>(smem + L.cbuf);
  uint32_t* grid = reinterpret_cast<uint32_t*>(smem + L.grid);  // (a << 16) | b
  int32_t* rowoff = reinterpret_cast<int32_t*>(smem + L.rowoff);
  __shared__ int s_gcount;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int st = blockIdx.y;
  const int h = st % a.H;
  const int t0 = blockIdx.x * kTT;
  const int dh = a.d_k / 2;
  uint64_t* buf = cbufs + wave * max(64, 2 * mmax);

  for (int pass = 0; pass < 2; pass++) {
    const void* X = pass == 0 ? a.kp : a.qp;
    const int k = pass == 0 ? a.W : a.R;
    const int m = k;  // stage-1 list length (k <= n_sub)
    const float z = pass == 0 ? zW : zR;
    int32_t* oidx = pass == 0 ? a.widx : a.ridx;
    float* owt = pass == 0 ? a.wwt : a.rwt;

    // pruned rank grid {(ra, rb) : (ra+1)(rb+1) <= k}, row-major; row
    // offsets by a prefix sum over wave 0 (m <= 128 rows, two per lane)
    if (wave == 0) {
      const int len0 = lane < m ? min(m, k / (lane + 1)) : 0;
      const int len1 = lane + 64 < m ? min(m, k / (lane + 65)) : 0;
      int s0 = len0, s1 = len1;
      for (int o = 1; o < 64; o <<= 1) {
        const int y0 = __shfl_up(s0, o), y1 = __shfl_up(s1, o);
        if (lane >= o) s0 += y0, s1 += y1;
      }
      const int tot0 = __shfl(s0, 63);
      const int G = tot0 + __shfl(s1, 63);
      if (lane < m) rowoff[lane] = s0 - len0;
      if (lane + 64 < m) rowoff[lane + 64] = tot0 + s1 - len1;
      if (lane == 0) rowoff[m] = G, s_gcount = G;
    }
    __syncthreads();
    for (int ra = wave; ra < m; ra += kWaves) {
      const int len = rowoff[ra + 1] - rowoff[ra];
      for (int rb = lane; rb < len; rb += 64) grid[rowoff[ra] + rb] = ((uint32_t)ra << 16) | rb;
    }

    for (int half = 0; half < 2; half++) {
      // ---- 1. half scores of the tile into sc[token][sub-key] -------------
      __syncthreads();  // previous users of sc are done
      if (BF16) {
        const int tl = lane & 15;
        const int tok = t0 + tl;
        const bool tok_ok = tl < kTT && tok < a.T;
        const uint16_t* Xb = static_cast<const uint16_t*>(X) +
                             ((int64_t)st * a.T + (tok_ok ? tok : 0)) * a.d_k + half * dh;
        const uint16_t* Cb = static_cast<const uint16_t*>(a.subkeys) +
                             ((int64_t)h * 2 + half) * n_sub * dh;
        if (dh <= 32) mfma_half_scores<1>(Xb, Cb, n_sub, dh, sc, scs, wave, lane, tok_ok);
        else if (dh <= 64) mfma_half_scores<2>(Xb, Cb, n_sub, dh, sc, scs, wave, lane, tok_ok);
        else if (dh <= 128) mfma_half_scores<4>(Xb, Cb, n_sub, dh, sc, scs, wave, lane, tok_ok);
        else mfma_half_scores<8>(Xb, Cb, n_sub, dh, sc, scs, wave, lane, tok_ok);
      } else {
        const float* Xf = static_cast<const float*>(X);
        const float* Cf = static_cast<const float*>(a.subkeys) +
                          ((int64_t)h * 2 + half) * n_sub * dh;
        for (int p = tid; p < kTT * n_sub; p += kThreads) {
          const int tl = p / n_sub, i = p % n_sub;
          const int tok = t0 + tl;
          if (tok >= a.T) continue;
          const float* x = Xf + ((int64_t)st * a.T + tok) * a.d_k + half * dh;
          const float* c = Cf + (int64_t)i * dh;
          sc[tl * scs + i] = dot_seq(x, c, dh);
        }
      }
      __syncthreads();

      // ---- 2. stage 1: top-m sub-keys of each token's half ----------------
      for (int tl = wave; tl < kTT; tl += kWaves) {
        if (t0 + tl >= a.T) continue;
        const float* row = sc + tl * scs;
        uint64_t key[NPL1];
        float sum = 0.f, sq = 0.f;
#pragma unroll
        for (int j = 0; j < NPL1; j++) {
          const int i = j * 64 + lane;
          if (i < n_sub) {
            const float s = row[i];
            key[j] = make_key(s, (uint32_t)i);
            sum += s;
            sq += s * s;
          } else {
            key[j] = 0ull;
          }
        }
        sum = wave_sum(sum);
        sq = wave_sum(sq);
        const float mean = sum / n_sub;
        const float sd = sqrtf(fmaxf(sq / n_sub - mean * mean, 0.f));
        const uint64_t guess = (uint64_t)ord32(mean + z * sd) << 32;
        float* ols = ls + (half * kTT + tl) * mmax;
        int32_t* oli = li + (half * kTT + tl) * mmax;
        wave_topk(key, m, guess, buf, lane, [&](int r, uint64_t kk) {
          ols[r] = key_score(kk);
          oli[r] = (int32_t)key_id(kk);
        });
      }
    }
    __syncthreads();  // both halves' lists complete

    // ---- 3. stage 2: top-k slots of the outer sums -------------------------
    const int G = s_gcount;
    for (int tl = wave; tl < kTT; tl += kWaves) {
      const int tok = t0 + tl;
      if (tok >= a.T) continue;
      const float* s1 = ls + (0 * kTT + tl) * mmax;
      const float* s2 = ls + (1 * kTT + tl) * mmax;
      const int32_t* i1 = li + (0 * kTT + tl) * mmax;
      const int32_t* i2 = li + (1 * kTT + tl) * mmax;
      uint64_t key[NPL2];
#pragma unroll
      for (int j = 0; j < NPL2; j++) {
        const int c = j * 64 + lane;
        key[j] = 0ull;
        if (c < G) {
          const uint32_t ab = grid[c];
          const int ra = ab >> 16, rb = ab & 0xffff;
          key[j] = make_key(s1[ra] + s2[rb], (uint32_t)(i1[ra] * n_sub + i2[rb]));
        }
      }
      // linear first guess between the extremes of the candidate scores
      uint64_t kth = 0ull;  // k-th best key of the pruned grid
      int32_t* dst_i = oidx + ((int64_t)st * a.T + tok) * k;
      float* dst_w = owt + ((int64_t)st * a.T + tok) * k;
      uint64_t* sorted = buf;  // reused below: sorted keys land here first
      {
        uint64_t mx = 0;
#pragma unroll
        for (int j = 0; j < NPL2; j++) mx = key[j] > mx ? key[j] : mx;
        mx = wave_max64(mx);
        const int cap = min(kCapMax, max(64, 2 * k));
        // first threshold: for any rank ra the rectangle [0..ra] x [0..cb] with
        // cb = ceil(k/(ra+1)) - 1 holds at least k sums, all at least its
        // corner's, so the best corner is a lower bound of the k-th sum
        uint64_t lb = 0ull;
        for (int ra = lane; ra < m; ra += 64) {
          const int cb = (k + ra) / (ra + 1) - 1;
          const uint64_t kk = (uint64_t)ord32(s1[ra] + s2[cb]) << 32;
          lb = kk > lb ? kk : lb;
        }
        lb = wave_max64(lb);
        const uint64_t t = find_threshold(key, k, cap, lb, 0ull, mx + 1ull);
        const int c = compact_ge(key, t, buf, lane);
        wave_lds_sync();
        // sort in place: emit writes back into buf positions < k
        sort_emit(buf, c, k, lane, [&](int r, uint64_t kk) { sorted[r] = kk; });
        wave_lds_sync();
        kth = sorted[k - 1];
      }
      // best pair just outside the pruned grid, row by row
      uint64_t fr = 0ull;
      for (int ra = lane; ra < m; ra += 64) {
        const int rb = min(m, k / (ra + 1));
        if (rb < m) {
          const uint64_t kk = make_key(s1[ra] + s2[rb], (uint32_t)(i1[ra] * n_sub + i2[rb]));
          fr = kk > fr ? kk : fr;
        }
      }
      fr = wave_max64(fr);
      // exact if no outside pair can outrank the k-th: compare scores only,
      // since a score tie with a lower slot would outrank it
      const bool exact = fr == 0ull || key_score(fr) < key_score(kth);
      if (!exact) {
        // rank the full m x m grid: keys >= kth are the candidates (at least
        // k of them); bisect upward if there are too many.
        const int cap = min(kCapMax, max(64, 2 * k));
        auto cnt = [&](uint64_t t) {
          int c = 0;
          for (int base = 0; base < m * m; base += 64) {
            const int q = base + lane;
            bool f = false;
            if (q < m * m) {
              const int ra = q / m, rb = q % m;
              f = make_key(s1[ra] + s2[rb], (uint32_t)(i1[ra] * n_sub + i2[rb])) >= t;
            }
            c += __popcll(__ballot(f));
          }
          return c;
        };
        uint64_t lo = kth, hi = ~0ull, t = kth;
        for (int it = 0; it < 96; it++) {
          const int c = cnt(t);
          if (c >= k && c <= cap) break;
          if (c < k) hi = t;
          else lo = t;
          if (hi - lo <= 1) {
            t = lo;
            break;
          }
          t = lo + (hi - lo) / 2;
        }
        int base = 0;
        const uint64_t below = (1ull << lane) - 1ull;
        for (int b0 = 0; b0 < m * m; b0 += 64) {
          const int q = b0 + lane;
          uint64_t kk = 0ull;
          if (q < m * m) {
            const int ra = q / m, rb = q % m;
            kk = make_key(s1[ra] + s2[rb], (uint32_t)(i1[ra] * n_sub + i2[rb]));
          }
          const bool f = q < m * m && kk >= t;
          const uint64_t msk = __ballot(f);
          if (f) buf[base + __popcll(msk & below)] = kk;
          base += __popcll(msk);
        }
        wave_lds_sync();
        sort_emit(buf, base, k, lane, [&](int r, uint64_t kk) { sorted[r] = kk; });
        wave_lds_sync();
      }
      // softmax over the k selected sums (rank order, max first)
      const float top = key_score(sorted[0]);
      float zsum = 0.f;
      for (int r = lane; r < k; r += 64) zsum += expf(key_score(sorted[r]) - top);
      zsum = wave_sum(zsum);
      for (int r = lane; r < k; r += 64) {
        const uint64_t kk = sorted[r];
        dst_i[r] = (int32_t)key_id(kk);
        dst_w[r] = expf(key_score(kk) - top) / zsum;
      }
      wave_lds_sync();
    }
    __syncthreads();  // lists and grid are rebuilt by the next pass
  }
}

// Inverse of the standard normal CDF (rational approximation, relative error
// about 1e-9; only steers the first threshold guess).
static inline double norm_quantile(double p) {
  static const double a[] = {-3.969683028665376e+01, 2.209460984245205e+02,
                             -2.759285104469687e+02, 1.383577518672690e+02,
                             -3.066479806614716e+01, 2.506628277459239e+00};
  static const double b[] = {-5.447609879822406e+01, 1.615858368580409e+02,
                             -1.556989798598866e+02, 6.680131188771972e+01,
                             -1.328068155288572e+01};
  static const double c[] = {-7.784894002430293e-03, -3.223964580411365e-01,
                             -2.400758277161838e+00, -2.549671010115749e+00,
                             4.374664141464968e+00, 2.938163982698783e+00};
  static const double d[] = {7.784695709041462e-03, 3.224671290700398e-01,
                             2.445134137142996e+00, 3.754408661907416e+00};
  if (p <= 0.0) return -8.0;
  if (p >= 1.0) return 8.0;
  const double pl = 0.02425;
  if (p < pl) {
    const double q = sqrt(-2 * log(p));
    return (((((c[0] * q + c[1]) * q + c[2]) * q + c[3]) * q + c[4]) * q + c[5]) /
           ((((d[0] * q + d[1]) * q + d[2]) * q + d[3]) * q + 1);
  }
  if (p > 1 - pl) {
    const double q = sqrt(-2 * log(1 - p));
    return -(((((c[0] * q + c[1]) * q + c[2]) * q + c[3]) * q + c[4]) * q + c[5]) /
           ((((d[0] * q + d[1]) * q + d[2]) * q + d[3]) * q + 1);
  }
  const double q = p - 0.5, r = q * q;
  return (((((a[0] * r + a[1]) * r + a[2]) * r + a[3]) * r + a[4]) * r + a[5]) * q /
         (((((b[0] * r + b[1]) * r + b[2]) * r + b[3]) * r + b[4]) * r + 1);
}

// threshold z such that about 1.4*k of n Gaussian scores lie above mean + z*sd
static inline float guess_z(int k, int n) {
  double f = 1.4 * k / n;
  if (f > 0.9) f = 0.9;
  return (float)norm_quantile(1.0 - f);
}

// size of the pruned rank grid {(a,b) : (a+1)(b+1) <= k} over k x k ranks
static inline int pruned_grid_size(int k) {
  int g = 0;
  for (int a = 0; a < k; a++) g += (k / (a + 1) < k ? k / (a + 1) : k);
  return g;
}

template <bool BF16, int NPL1, int NPL2>
static inline hipError_t launch_t(const ScoreArgs& a, hipStream_t stream) {
  const ScoreSmem L = score_smem(a.n_sub, a.W > a.R ? a.W : a.R);
  auto k = sdm_score_topk_kernel<BF16, NPL1, NPL2>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)L.total);
  if (e != hipSuccess) return e;
  dim3 grid((a.T + kTT - 1) / kTT, a.S);
  hipLaunchKernelGGL(k, grid, dim3(kThreads), L.total, stream, a, guess_z(a.W, a.n_sub),
                     guess_z(a.R, a.n_sub));
  return hipGetLastError();
}

// Launch for one stage-1 width NPL1 (scores per lane), any stage-2 width.
template <int NPL1>
hipError_t launch_score_n(const ScoreArgs& a, bool bf16, int npl2, hipStream_t stream) {
#define SDM_SCORE_CASE(M_)                                                      \
  if (npl2 <= M_) return bf16 ? launch_t<true, NPL1, M_>(a, stream) : launch_t<false, NPL1, M_>(a, stream);
  SDM_SCORE_CASE(4)
  SDM_SCORE_CASE(8)
  SDM_SCORE_CASE(12)
  SDM_SCORE_CASE(16)
#undef SDM_SCORE_CASE
  return hipErrorInvalidValue;
}

}  // namespace sdm
